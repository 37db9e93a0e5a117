"""GPU parity of paged_attn_prefill_varlen (and the mixed ragged step) against the oracle."""

import numpy as np
import pytest
import torch

import paged_kv_flashattention_amd as pa
import oracle
from tests.parity import (as_f64, assert_lse, assert_parity, oracle_by_sequence, oracle_full,
                          oracle_rows, pools_after_write)
from workloads import bits, make_case, make_config

pytestmark = pytest.mark.gpu


def write(case):
    if case.k_new is not None:
        pa.kv_page_write(case.k_pool, case.v_pool, case.k_new, case.v_new, case.cu_new,
                         case.start_pos, case.block_tables, validate=True)


def run_prefill(case, causal=None):
    out, lse = pa.paged_attn_prefill_varlen(
        case.q, case.k_pool, case.v_pool, case.cu_seqlens_q, case.seq_lens_k, case.block_tables,
        case.scale, causal=case.causal if causal is None else causal, max_q_len=case.max_q_len,
        return_lse=True, validate=True)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    # hist, q_lens, Hq, Hkv, D, ps, causal
    ([0], [1], 4, 1, 128, 16, True),
    ([0, 0], [127, 300], 8, 2, 128, 16, True),
    ([200, 31, 0], [129, 1, 64], 8, 2, 128, 16, True),     # chunks over history
    ([1000, 0], [100, 257], 28, 4, 128, 16, True),         # GQA 7
    ([64, 5], [70, 33], 16, 1, 128, 64, True),             # GQA 16, page 64
    ([17, 0], [50, 130], 8, 8, 64, 32, True),              # MHA, D 64, page 32
    ([300, 0, 7], [40, 129, 1], 8, 2, 128, 16, False),     # non-causal
    ([0, 0], [1, 2], 4, 2, 64, 16, False),
    # max_q_len >= 512: 256-row work-groups (8 waves), ragged last tiles
    ([0, 0], [1100, 300], 4, 2, 64, 16, True),
    ([500, 0], [1030, 260], 8, 2, 128, 32, True),
    ([0], [1024], 4, 4, 128, 64, False),
    # the 256-row threshold itself: 511 rows (4 waves) and 512 rows (8 waves)
    ([40, 0], [511, 77], 8, 2, 128, 16, True),
    ([0, 40], [512, 77], 8, 2, 128, 16, True),
    # 8 waves with GQA 16 and D 64 (page 32), and without the causal mask
    ([0, 300], [700, 40], 16, 1, 64, 32, True),
    ([250, 0], [600, 513], 8, 4, 128, 16, False),
]


@pytest.mark.parametrize("hist,ql,Hq,Hkv,D,ps,causal", CASES)
def test_prefill_small(require_gpu, hist, ql, Hq, Hkv, D, ps, causal):
    print(f"[prefill] hist={hist} q={ql} Hq={Hq} Hkv={Hkv} D={D} ps={ps} causal={causal}",
          flush=True)
    case = make_case("pf", hist_lens=hist, q_lens=ql, write_new=True, causal=causal, Hq=Hq,
                     Hkv=Hkv, D=D, page_size=ps, seed=sum(ql) + Hq, device="cuda",
                     num_pages=sum(-(-(h + n) // ps) for h, n in zip(hist, ql)) + 2)
    kp, vp = pools_after_write(case)
    write(case)
    out, lse = run_prefill(case)
    o_ref, l_ref = oracle_full(case, kp, vp)
    assert_parity(as_f64(out), o_ref, "prefill")
    assert_lse(as_f64(lse), l_ref, "prefill lse")


def test_prefill_extreme_logits(require_gpu):
    case = make_case("pfx", hist_lens=[100, 0], q_lens=[200, 65], write_new=True, causal=True,
                     Hq=8, Hkv=2, D=128, page_size=16, seed=77, device="cuda")
    case.q = (case.q.float() * 30).to(torch.bfloat16)
    kp, vp = pools_after_write(case)
    write(case)
    out, lse = run_prefill(case)
    o_ref, l_ref = oracle_full(case, kp, vp)
    assert_parity(as_f64(out), o_ref, "prefill extreme")
    assert_lse(as_f64(lse), l_ref, "prefill extreme lse")


def test_prefill_decode_rows_match_decode_kernel(require_gpu):
    """q_len = 1 rows through the prefill kernel agree with the decode kernel."""
    case = make_case("pd", seq_lens=[1, 500, 4096, 17], q_lens=[1, 1, 1, 1], Hq=32, Hkv=8, D=128,
                     page_size=16, seed=21, causal=True, device="cuda")
    out_p, _ = run_prefill(case)
    out_d = pa.paged_attn_decode(case.q, case.k_pool, case.v_pool, case.block_tables,
                                 case.seq_lens_k, case.scale, max_seq_len=4096)
    o_ref, _ = oracle_full(case)
    assert_parity(as_f64(out_p), o_ref, "prefill q_len=1")
    assert_parity(as_f64(out_d), o_ref, "decode")


def _head_rows_oracle(case, kp, vp, b, h):
    """Every row of query head h of sequence b from the oracle, run on that sequence's
    pages and the KV head h reads (compact pool, table 0 .. n-1, Hq = Hkv = 1)."""
    bt = case.block_tables.cpu().numpy()
    cu = case.cu_seqlens_q.cpu().numpy()
    L = case.seq_lens[b]
    n = -(-L // case.page_size)
    kvh = h // (case.Hq // case.Hkv)
    pages = bt[b, :n].astype(np.int64)
    t0, t1 = int(cu[b]), int(cu[b + 1])
    o, ls = oracle.attention_ref(bits(case.q)[t0:t1, h:h + 1],
                                 np.ascontiguousarray(kp[pages][:, :, kvh:kvh + 1]),
                                 np.ascontiguousarray(vp[pages][:, :, kvh:kvh + 1]),
                                 np.arange(n, dtype=np.int32)[None], [L], [0, t1 - t0],
                                 case.scale, True, case.page_size)
    return o[:, 0], ls[:, 0]


def test_causal_prefill_full_size_every_work_group(require_gpu):
    """Dense causal prefill at full size: 4 x 4096 tokens, Hq 32, Hkv 8, written via
    kv_page_write then attended in the launch the benchmark times.  The oracle checks
    one complete query head per (sequence, KV head) -- 32 heads of 4,096 rows, every
    query tile and key tile of their groups -- and one row of every other (head,
    sequence, 128-row query block), so every work-group of the grid (2,048 of them,
    each two heads' 128 rows with paired heads, or one head's 256) has rows checked."""
    case = make_config("causal_prefill", "cuda")
    print("[prefill] causal_prefill full size, every work-group", flush=True)
    kp, vp = pools_after_write(case)
    write(case)
    assert np.array_equal(bits(case.k_pool), kp)
    out, lse = run_prefill(case)
    G = case.Hq // case.Hkv
    got, ref, got_l, ref_l = [], [], [], []
    whole = {(b, kvh * G + (b + 3 * kvh) % G) for b in range(case.B) for kvh in range(case.Hkv)}
    for b, h in sorted(whole):
        o, ls = _head_rows_oracle(case, kp, vp, b, h)
        got.append(as_f64(out[4096 * b:4096 * (b + 1), h]))
        got_l.append(as_f64(lse[4096 * b:4096 * (b + 1), h]))
        ref.append(o)
        ref_l.append(ls)
    rng = np.random.default_rng(5)
    rows = []
    for b in range(case.B):
        for h in range(case.Hq):
            if (b, h) in whole:
                continue
            for qt in range(4096 // 128):
                rows.append((4096 * b + 128 * qt + int(rng.integers(0, 128)), h))
    o_ref, l_ref = oracle_rows(case, rows, kp, vp)
    idx_t = torch.as_tensor([t for t, _ in rows], device="cuda")
    idx_h = torch.as_tensor([h for _, h in rows], device="cuda")
    got.append(as_f64(out[idx_t, idx_h]))
    got_l.append(as_f64(lse[idx_t, idx_h]))
    ref.append(o_ref)
    ref_l.append(l_ref)
    assert_parity(np.concatenate(got), np.concatenate(ref), "causal_prefill")
    assert_lse(np.concatenate(got_l), np.concatenate(ref_l), "causal_prefill lse")
    assert torch.isfinite(out.float()).all()


def run_prefill_splitk(case, splits, causal=None, workspace=None):
    out, lse = pa.paged_attn_prefill_varlen_splitk(
        case.q, case.k_pool, case.v_pool, case.cu_seqlens_q, case.seq_lens_k, case.block_tables,
        case.scale, causal=case.causal if causal is None else causal, max_q_len=case.max_q_len,
        num_splits=splits, workspace=workspace, return_lse=True, validate=True)
    torch.cuda.synchronize()
    return out, lse


SPLIT_CASES = [
    # hist, q_lens, Hq, Hkv, D, ps, causal, splits
    ([4113, 214, 0], [512, 512, 40], 8, 2, 128, 16, True, 3),     # one long history
    ([3000, 0], [100, 1], 4, 1, 128, 16, True, 0),                # automatic: 8 parts at most
    ([2500, 9], [300, 20], 8, 8, 64, 32, False, 4),               # non-causal, D 64
    ([1500, 2200], [1100, 64], 4, 2, 128, 64, True, 2),           # 256-row work-groups
    ([0], [3000], 4, 2, 128, 16, True, 16),                       # no history, 16 parts at most
    ([5000], [1], 8, 1, 128, 16, True, 5),                        # a decode row, GQA 8
]


@pytest.mark.parametrize("hist,ql,Hq,Hkv,D,ps,causal,splits", SPLIT_CASES)
def test_prefill_splitk_parity(require_gpu, hist, ql, Hq, Hkv, D, ps, causal, splits):
    print(f"[prefill splitk] hist={hist} q={ql} Hq={Hq} Hkv={Hkv} D={D} ps={ps} "
          f"causal={causal} S={splits}", flush=True)
    case = make_case("pfs", hist_lens=hist, q_lens=ql, write_new=True, causal=causal, Hq=Hq,
                     Hkv=Hkv, D=D, page_size=ps, seed=sum(hist) + sum(ql) + Hq, device="cuda",
                     num_pages=sum(-(-(h + n) // ps) for h, n in zip(hist, ql)) + 2)
    kp, vp = pools_after_write(case)
    write(case)
    out, lse = run_prefill_splitk(case, splits)
    desc = pa.describe_launch()
    assert "prefill_merge" in desc, desc          # some tile was split
    o_ref, l_ref = oracle_full(case, kp, vp)
    assert_parity(as_f64(out), o_ref, "prefill splitk")
    assert_lse(as_f64(lse), l_ref, "prefill splitk lse")


def test_prefill_splitk_unsplit_tiles_are_bitwise_the_plain_prefill(require_gpu):
    """One part per tile (S = 1, or tiles shorter than two parts) is the plain launch."""
    case = make_case("pfb", hist_lens=[700, 0, 31], q_lens=[129, 300, 5], write_new=True,
                     causal=True, Hq=8, Hkv=2, D=128, page_size=16, seed=12, device="cuda")
    write(case)
    ref, lref = run_prefill(case)
    for splits in (1, 4):
        out, lse = run_prefill_splitk(case, splits)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), splits
        assert torch.equal(lse, lref), splits


def test_prefill_splitk_workspace_is_scratch(require_gpu):
    """A garbage-filled workspace, reused by two calls of different shapes, gives the
    oracle's result both times."""
    ws = torch.full((64 << 20,), 0xFF, dtype=torch.uint8, device="cuda")
    for i, (hist, ql) in enumerate([([4000, 10], [64, 3]), ([2100], [700])]):
        case = make_case("pfw", hist_lens=hist, q_lens=ql, write_new=True, causal=True, Hq=8,
                         Hkv=2, D=128, page_size=16, seed=30 + i, device="cuda")
        kp, vp = pools_after_write(case)
        write(case)
        out, lse = run_prefill_splitk(case, 4, workspace=ws)
        o_ref, l_ref = oracle_full(case, kp, vp)
        assert_parity(as_f64(out), o_ref, f"prefill splitk ws {i}")
        assert_lse(as_f64(lse), l_ref, f"prefill splitk ws lse {i}")


def test_long_history_chunk_full_size(require_gpu):
    """A 512-token chunk over a 32,768-token history (Hq 32, Hkv 8), with the library's
    own key-part count as the benchmark runs it; every row against the oracle."""
    case = make_config("long_history_chunk", "cuda")
    print("[prefill splitk] long_history_chunk full size, every row", flush=True)
    kp, vp = pools_after_write(case)
    write(case)
    assert pa.prefill_num_splits(1, 32, 512) > 1
    out, lse = run_prefill_splitk(case, 0)
    assert "prefill_merge" in pa.describe_launch()
    o_ref, l_ref = oracle_by_sequence(case, kp, vp, split_kv_heads=True)
    assert_parity(as_f64(out), o_ref, "long_history_chunk")
    assert_lse(as_f64(lse), l_ref, "long_history_chunk lse")


@pytest.mark.parametrize("splitk", [0, 4, -1])
def test_mixed_ragged_step_full_size(require_gpu, splitk):
    """The mixed step: write all 2,578 new tokens, prefill the five 512-token chunks over
    their history (in one pass, or with long key ranges split into 4 parts or into the
    host planner's count, and merged), decode the 18 single-token requests, all on the
    same pools."""
    case = make_config("mixed_ragged", "cuda")
    n_pf = 5
    if splitk < 0:
        splitk = pa.prefill_plan_splits(case.q_lens[:n_pf], case.seq_lens[:n_pf], case.Hq)
    print(f"[mixed] mixed_ragged full size, splitk={splitk}", flush=True)
    kp, vp = pools_after_write(case)
    write(case)
    cu = case.cu_seqlens_q
    t_pf = int(cu[n_pf])
    extra = dict(num_splits=splitk) if splitk else {}
    prefill = pa.paged_attn_prefill_varlen_splitk if splitk else pa.paged_attn_prefill_varlen
    out_p, lse_p = prefill(
        case.q[:t_pf], case.k_pool, case.v_pool, cu[:n_pf + 1].contiguous(),
        case.seq_lens_k[:n_pf].contiguous(), case.block_tables[:n_pf].contiguous(), case.scale,
        causal=True, max_q_len=512, return_lse=True, validate=True, **extra)
    if splitk:
        assert "prefill_merge" in pa.describe_launch()
    out_d, lse_d = pa.paged_attn_decode(
        case.q[t_pf:].contiguous(), case.k_pool, case.v_pool,
        case.block_tables[n_pf:].contiguous(), case.seq_lens_k[n_pf:].contiguous(), case.scale,
        max_seq_len=max(case.seq_lens[n_pf:]), return_lse=True, validate=True)
    torch.cuda.synchronize()
    # every row of the step: the 2,560 prefill rows and the 18 decode rows, all heads
    o_ref, l_ref = oracle_by_sequence(case, kp, vp)
    got = np.concatenate([as_f64(out_p), as_f64(out_d)])
    got_l = np.concatenate([as_f64(lse_p), as_f64(lse_d)])
    assert_parity(got, o_ref, "mixed step")
    assert_lse(got_l, l_ref, "mixed lse")


@pytest.mark.parametrize("hist,ql", [
    # 256-row tiles (a run of >= 512): rows ending at every offset within a wave's 32
    # and a block's 32 keys, waves with no valid row, with and without history
    ([0, 0, 0, 0], [1024, 31, 33, 257]),
    ([0, 5, 64], [1025, 63, 65]),
    ([100, 0], [1100, 1]),
    # 128-row tiles
    ([0, 0, 0], [129, 32, 95]),
    ([37, 0], [200, 64]),
])
def test_causal_prefill_rows_ending_mid_tile(require_gpu, hist, ql):
    """Causal rows whose last key falls anywhere in a tile: each wave computes only
    the blocks up to its last valid row (the rest of its tiles it only moves), so
    every (tile size, row offset, history) combination is checked against the oracle."""
    print(f"[prefill causal tail] hist={hist} q={ql}", flush=True)
    case = make_case("pft", hist_lens=hist, q_lens=ql, write_new=True, causal=True, Hq=8,
                     Hkv=2, D=128, page_size=16, seed=sum(ql) + 77, device="cuda")
    kp, vp = pools_after_write(case)
    write(case)
    out, lse = run_prefill(case)
    o_ref, l_ref = oracle_full(case, kp, vp)
    assert_parity(as_f64(out), o_ref, "prefill causal tail")
    assert_lse(as_f64(lse), l_ref, "prefill causal tail lse")


@pytest.mark.parametrize("hist,ql,Hq,Hkv,classes", [
    ([0, 100], [1100, 300], 8, 2, 2),     # 4 groups: 2 rank classes, 5 tiles (one surplus)
    ([0, 0, 7], [800, 5, 300], 12, 2, 4), # 6 groups: 4 classes would be needed -> head-major
])
def test_prefill_xcd_rank_classes(require_gpu, hist, ql, Hq, Hkv, classes):
    """A group count that is not a multiple of 8: an even one deals each group's
    query-tile ranks into 2 classes on 2 XCDs (every tile computed exactly once, the
    surplus work-groups of an odd tile count return at once); otherwise head-major."""
    print(f"[prefill xcd classes] hist={hist} q={ql} Hq={Hq} Hkv={Hkv}", flush=True)
    case = make_case("pxc", hist_lens=hist, q_lens=ql, write_new=True, causal=True, Hq=Hq,
                     Hkv=Hkv, D=128, page_size=16, seed=61, device="cuda")
    kp, vp = pools_after_write(case)
    write(case)
    out, lse = run_prefill(case)
    desc = pa.describe_launch()
    if classes == 2:
        assert "2 rank classes" in desc, desc
    else:
        assert "head-major" in desc, desc
    o_ref, l_ref = oracle_full(case, kp, vp)
    assert_parity(as_f64(out), o_ref, "prefill xcd classes")
    assert_lse(as_f64(lse), l_ref, "prefill xcd classes lse")


NO_KEY_CASES = [
    # seq_lens (keys), q_lens, causal, splits, window, alibi
    ([0, 10, 300], [37, 50, 20], True, 1, 0, False),         # 4 waves: L = 0, L < q_len
    ([0, 7], [5, 9], False, 1, 0, False),                    # non-causal, L = 0
    ([100, 0], [600, 3], True, 1, 0, False),                 # 8 waves: 500 rows see nothing
    ([0, 3000, 2500], [20, 3100, 300], True, 4, 0, False),   # key parts over L < q_len
    ([0, 40], [30, 100], True, 1, 64, True),                 # window + ALiBi variant
    ([0, 700], [10, 900], True, 1, 0, True),                 # ALiBi, 8 waves, walked down
]


@pytest.mark.parametrize("lens,ql,causal,splits,window,alibi", NO_KEY_CASES)
def test_prefill_rows_that_see_no_key(require_gpu, lens, ql, causal, splits, window, alibi):
    """Rows of a sequence with no keys, or causal rows placed before the sequence's
    first key (q_len > keys, bottom-right alignment), give exactly O = 0 and lse = -inf
    ("8. Kernels and Attention Backends", "Test the kernel at three levels": a fully
    masked row needs a defined value); every other row matches the oracle."""
    print(f"[prefill no-key] lens={lens} q={ql} causal={causal} S={splits} w={window} "
          f"alibi={alibi}", flush=True)
    case = make_case("pnk", seq_lens=lens, q_lens=ql, causal=causal, Hq=8, Hkv=2, D=128,
                     page_size=16, seed=sum(lens) + sum(ql), device="cuda", window=window,
                     num_pages=sum(-(-L // 16) for L in lens) + 3)
    slopes = None
    if alibi:
        slopes = torch.tensor([2.0 ** (-(h + 1)) for h in range(8)], dtype=torch.float32,
                              device="cuda")
    if splits > 1:
        out, lse = pa.paged_attn_prefill_varlen_splitk(
            case.q, case.k_pool, case.v_pool, case.cu_seqlens_q, case.seq_lens_k,
            case.block_tables, case.scale, causal=causal, max_q_len=case.max_q_len,
            num_splits=splits, return_lse=True, validate=True, window_left=window,
            alibi_slopes=slopes)
        assert "prefill_merge" in pa.describe_launch()
    else:
        out, lse = pa.paged_attn_prefill_varlen(
            case.q, case.k_pool, case.v_pool, case.cu_seqlens_q, case.seq_lens_k,
            case.block_tables, case.scale, causal=causal, max_q_len=case.max_q_len,
            return_lse=True, validate=True, window_left=window, alibi_slopes=slopes)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_full(case, bits(case.k_pool), bits(case.v_pool),
                               alibi=None if slopes is None else slopes.cpu().numpy())
    empty = np.isneginf(l_ref)
    assert empty.any()
    got_o, got_l = as_f64(out), as_f64(lse)
    assert (got_o[empty] == 0).all(), "a row with no key has a nonzero output"
    assert np.isneginf(got_l[empty]).all(), "a row with no key has a finite lse"
    assert_parity(got_o, o_ref, "prefill no-key")
    assert_lse(got_l, l_ref, "prefill no-key lse")


PAIR_CASES = [
    # hist, q_lens, Hq, Hkv, D, causal
    ([0, 0, 0], [1024, 129, 600], 8, 4, 128, True),        # GQA 2
    ([300, 0], [700, 512], 16, 1, 128, True),              # GQA 16
    ([0, 64], [513, 900], 32, 4, 64, True),                # GQA 8, D 64
    ([1000, 0], [530, 1100], 8, 2, 128, False),            # non-causal
    ([0, 0], [1030, 520], 28, 4, 128, True),               # GQA 7: one head per work-group
]


@pytest.mark.parametrize("hist,ql,Hq,Hkv,D,causal", PAIR_CASES)
def test_paired_heads_give_the_256_row_bits(require_gpu, hist, ql, Hq, Hkv, D, causal):
    """An unsplit 8-wave launch with an even GQA group pairs two query heads over 128 rows
    per work-group; the output bits equal the 256-row layout's (taken from the
    persistent grid, which keeps it) and match the oracle; an odd group keeps one head
    per work-group."""
    print(f"[paired heads] hist={hist} q={ql} Hq={Hq} Hkv={Hkv} D={D} causal={causal}",
          flush=True)
    case = make_case("php", hist_lens=hist, q_lens=ql, write_new=True, causal=causal, Hq=Hq,
                     Hkv=Hkv, D=D, page_size=16, seed=sum(ql) + Hq, device="cuda")
    kp, vp = pools_after_write(case)
    write(case)
    o0, l0 = run_prefill(case)
    desc = pa.describe_launch()
    assert ("paired heads" in desc) == ((Hq // Hkv) % 2 == 0), desc
    o1, l1 = pa.paged_attn_prefill_varlen(
        case.q, case.k_pool, case.v_pool, case.cu_seqlens_q, case.seq_lens_k, case.block_tables,
        case.scale, causal=causal, max_q_len=case.max_q_len, return_lse=True, persistent=True)
    torch.cuda.synchronize()
    assert "BM=256" in pa.describe_launch()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l0.view(torch.int32), l1.view(torch.int32))
    o_ref, l_ref = oracle_full(case, kp, vp)
    assert_parity(as_f64(o0), o_ref, "paired heads")
    assert_lse(as_f64(l0), l_ref, "paired heads lse")
