"""GPU parity of paged_attn_decode (+ its split-K reduce) against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_flashattention_amd as pa
from tests.parity import (as_f64, assert_lse, assert_parity, oracle_by_sequence, oracle_full,
                          oracle_rows, pools_after_write)
from workloads import bits, make_case, make_config, units

pytestmark = pytest.mark.gpu


def run_decode(case, num_splits=0, max_seq_len=None):
    out, lse = pa.paged_attn_decode(case.q, case.k_pool, case.v_pool, case.block_tables,
                                    case.seq_lens_k, case.scale,
                                    max_seq_len=case.max_seq_len if max_seq_len is None else max_seq_len,
                                    num_splits=num_splits, return_lse=True, validate=True)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("splits", [1, 2, 3, 8, 0, 64])
def test_tiny_decode_config(require_gpu, splits):
    case = make_config("tiny_decode", "cuda")
    print(f"[decode] tiny_decode splits={splits}", flush=True)
    out, lse = run_decode(case, splits)
    o_ref, l_ref = oracle_full(case)
    assert_parity(as_f64(out), o_ref, "tiny_decode")
    assert_lse(as_f64(lse), l_ref, "tiny_decode lse")


AWKWARD = [
    # seq_lens, Hq, Hkv, D, ps, splits
    ([1, 15, 16, 17], 8, 2, 128, 16, 1),
    ([1, 15, 16, 17], 8, 2, 128, 16, 4),
    ([127, 4096, 33, 64], 28, 4, 128, 16, 0),
    ([127, 4096, 33, 64], 28, 4, 128, 16, 7),
    ([0, 5, 0, 300], 32, 8, 128, 16, 3),
    ([200, 1000], 16, 1, 128, 64, 5),         # GQA 16, page size 64
    ([200, 1000], 8, 8, 64, 32, 2),           # MHA, D 64, page size 32
    ([513, 77, 1], 7, 1, 64, 64, 0),          # GQA 7, D 64
    ([100], 4, 4, 128, 16, 64),               # more splits than chunks
    # >= 512 work-groups (one wave each) and 256 (two waves each)
    ([(37 * i) % 701 for i in range(64)], 16, 8, 128, 16, 1),
    ([(37 * i) % 701 for i in range(64)], 16, 8, 128, 16, 2),
    ([(53 * i) % 509 for i in range(64)], 8, 8, 64, 16, 2),
    ([(91 * i) % 1201 for i in range(32)], 32, 8, 64, 32, 1),
]


@pytest.mark.parametrize("lens,Hq,Hkv,D,ps,splits", AWKWARD)
def test_awkward_shapes(require_gpu, lens, Hq, Hkv, D, ps, splits):
    print(f"[decode] awkward lens={lens} Hq={Hq} Hkv={Hkv} D={D} ps={ps} S={splits}", flush=True)
    case = make_case("awk", seq_lens=lens, Hq=Hq, Hkv=Hkv, D=D, page_size=ps, seed=sum(lens) + D,
                     num_pages=sum(-(-L // ps) for L in lens) + 5, device="cuda")
    out, lse = run_decode(case, splits)
    o_ref, l_ref = oracle_full(case)
    assert_parity(as_f64(out), o_ref, "awkward")
    assert_lse(as_f64(lse), l_ref, "awkward lse")
    for b, L in enumerate(lens):
        if L == 0:       # no key: defined zeros, lse = -inf
            assert (as_f64(out[b]) == 0).all()
            assert np.isneginf(as_f64(lse[b])).all()


def test_extreme_logits(require_gpu):
    case = make_case("x", seq_lens=[700, 33, 4096], Hq=28, Hkv=4, D=128, page_size=16, seed=5,
                     device="cuda")
    case.q = (case.q.float() * 30).to(torch.bfloat16)
    print("[decode] extreme logits", flush=True)
    out, lse = run_decode(case, 4)
    o_ref, l_ref = oracle_full(case)
    assert_parity(as_f64(out), o_ref, "extreme logits")
    assert_lse(as_f64(lse), l_ref, "extreme lse")


@pytest.mark.parametrize("splits", [1, 5])
def test_dominant_key_gathers_bit_exact(require_gpu, splits):
    """Each query matches one key so strongly that every other weight underflows to 0
    in fp32: the output must be that key's V row exactly (pins page/slot indexing)."""
    lens = [300, 77, 1024]
    case = make_case("dom", seq_lens=lens, Hq=8, Hkv=2, D=128, page_size=16, seed=9,
                     device="cuda", std_kv=0.01)
    rng = np.random.default_rng(0)
    targets = [int(rng.integers(0, L)) for L in lens]
    bt = case.block_tables.cpu().numpy()
    for b, j in enumerate(targets):
        page, slot = int(bt[b, j // 16]), j % 16
        for kvh in range(2):
            case.k_pool[page, slot, kvh] = 0
            case.k_pool[page, slot, kvh, 0] = 64.0
    case.q.zero_()
    case.q[:, :, 0] = 64.0   # score gap 64 * 64 / sqrt(128) ~ 362 >> 110
    print(f"[decode] dominant key splits={splits}", flush=True)
    out, _ = run_decode(case, splits)
    vp = bits(case.v_pool)
    got = bits(out)
    for b, j in enumerate(targets):
        page, slot = int(bt[b, j // 16]), j % 16
        for h in range(8):
            assert np.array_equal(got[b, h], vp[page, slot, h // 4]), (b, h)


def test_single_key_returns_value_row_bit_exact(require_gpu):
    case = make_case("one", seq_lens=[1, 1, 1], Hq=16, Hkv=4, D=128, page_size=16, seed=3,
                     device="cuda")
    out, lse = run_decode(case, 1)
    vp = bits(case.v_pool)
    bt = case.block_tables.cpu().numpy()
    got = bits(out)
    for b in range(3):
        for h in range(16):
            assert np.array_equal(got[b, h], vp[bt[b, 0], 0, h // 4])


def test_repeat_runs_are_bitwise_identical(require_gpu):
    case = make_case("det", seq_lens=[3000, 17, 999, 4096], Hq=28, Hkv=4, D=128, page_size=16,
                     seed=4, device="cuda")
    ref = bits(run_decode(case, 6)[0])
    for _ in range(20):
        assert np.array_equal(bits(run_decode(case, 6)[0]), ref)


@pytest.mark.parametrize("S,D", [(9, 128), (2, 128), (3, 64), (5, 128), (8, 64), (70, 128)])
def test_splitk_reduce_standalone_matches_merge(require_gpu, S, D):
    """Both merge paths: all loads of a row at once (S <= 8) and the general one."""
    rng = np.random.default_rng(11 + S)
    R = 37
    po = rng.standard_normal((R, S, D)).astype(np.float32)
    pl = (rng.standard_normal((R, S)) * 5).astype(np.float32)
    pl[3, :] = -np.inf           # a row with every partition empty
    pl[4, ::2] = -np.inf         # some empty partitions
    out, lse = pa.paged_attn_splitk_reduce(torch.as_tensor(po, device="cuda"),
                                           torch.as_tensor(pl, device="cuda"))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.merge_ref(po.astype(np.float64), pl.astype(np.float64))
    # the merge is fp32 and its output bf16: each element within bf16's relative
    # rounding (2^-9, doubled for the fp32 sums) of the exact merge
    err = np.abs(as_f64(out) - o_ref)
    assert (err <= np.abs(o_ref) * 2.0 ** -8 + 1e-5).all(), float(err.max())
    assert_parity(as_f64(out), o_ref, "reduce", max_abs=2e-2, mean_abs=2e-3)
    assert_lse(as_f64(lse), l_ref, "reduce lse")
    assert (as_f64(out[3]) == 0).all()
    assert ("_few" in pa.describe_launch()) == (S <= 8)


def test_qwen7b_decode_full_size(require_gpu):
    """Qwen2.5-7B-shaped decode at its full size (32 x 8192, Hq 28, Hkv 4), in the
    launch configuration the benchmark times (the library's split count); every one
    of the 896 (sequence, head) rows against the oracle."""
    case = make_config("qwen7b_decode", "cuda")
    print("[decode] qwen7b full size, every row", flush=True)
    out, lse = run_decode(case, 0)
    o_ref, l_ref = oracle_by_sequence(case, bits(case.k_pool), bits(case.v_pool))
    assert_parity(as_f64(out), o_ref, "qwen7b full")
    assert_lse(as_f64(lse), l_ref, "qwen7b lse")


@pytest.mark.parametrize("splits", [64, 0])
def test_long_context_decode_full_size(require_gpu, splits):
    """Long-context decode at full size (8 x 131072, Hq 64, Hkv 8, page 64) with the 64
    partitions it is stated with (4,096 one-wave work-groups) and with the library's
    own split count; every one of the 512 (sequence, head) rows against the oracle,
    which takes one sequence's pages and one KV head at a time."""
    case = make_config("long_decode", "cuda")
    print(f"[decode] long_decode full size, every row, splits={splits}", flush=True)
    out, lse = run_decode(case, splits)
    o_ref, l_ref = oracle_by_sequence(case, bits(case.k_pool), bits(case.v_pool),
                                      split_kv_heads=True)
    assert_parity(as_f64(out), o_ref, "long_decode full")
    assert_lse(as_f64(lse), l_ref, "long lse")


def test_workspace_is_scratch_and_reusable(require_gpu):
    """A workspace full of garbage, reused across calls with different split counts and
    batch shapes, gives the oracle's result every time."""
    cases = [make_case("ws", seq_lens=lens, Hq=28, Hkv=4, D=128, page_size=16, seed=40 + i,
                       device="cuda")
             for i, lens in enumerate([[3000, 17, 999, 4096], [8192] * 3, [77]])]
    ws = torch.randint(0, 256, (64 << 20,), dtype=torch.uint8, device="cuda")   # garbage
    refs = [oracle_full(c)[0] for c in cases]
    for rep in range(2):
        for i, c in enumerate(cases):
            for S in (2, 5, 16):
                out = pa.paged_attn_decode(c.q, c.k_pool, c.v_pool, c.block_tables,
                                           c.seq_lens_k, c.scale, max_seq_len=c.max_seq_len,
                                           num_splits=S, workspace=ws)
                torch.cuda.synchronize()
                assert_parity(as_f64(out), refs[i], f"case {i} S={S} rep {rep}")


def test_graph_replays_match_eager(require_gpu):
    """A captured split-K decode (partition + merge launches) replayed several times,
    with eager work and synchronisations between replays, matches the eager result on
    every replay."""
    case = make_case("g", seq_lens=[5000, 3000, 8192, 100], Hq=28, Hkv=4, D=128, page_size=16,
                     seed=50, device="cuda")
    S = 4
    need = pa.decode_workspace_bytes(case.B, case.Hq, case.Hkv, case.D, 8192, S)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.empty((case.B, case.Hq, case.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((case.B, case.Hq), dtype=torch.float32, device="cuda")
    args = (case.q, case.k_pool, case.v_pool, case.block_tables, case.seq_lens_k, case.scale)
    pa.paged_attn_decode(*args, max_seq_len=8192, num_splits=S, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    ref_o, ref_l = bits(out).copy(), lse.cpu().numpy().copy()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pa.paged_attn_decode(*args, max_seq_len=8192, num_splits=S, out=out, lse=lse,
                                 workspace=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), ref_o), rep
        assert np.array_equal(lse.cpu().numpy(), ref_l), rep
        # eager work with the same workspace between replays
        pa.paged_attn_decode(*args, max_seq_len=8192, num_splits=3, workspace=ws)
        torch.cuda.synchronize()


@pytest.mark.parametrize("lens,S", [([3000, 17, 999, 4096], 4), ([100, 0, 64], 3), ([8192], 1)])
def test_partials_match_oracle_chunks_and_merge_to_decode(require_gpu, lens, S):
    """decode_partials gives each partition's own attention and lse (the oracle's
    per-chunk partials over the same boundaries), and reducing them reproduces
    paged_attn_decode bit for bit."""
    case = make_case("parts", seq_lens=lens, Hq=28, Hkv=4, D=128, page_size=16, seed=60 + S,
                     device="cuda")
    max_len = max(lens)
    po, pl = pa.paged_attn_decode_partials(case.q, case.k_pool, case.v_pool, case.block_tables,
                                           case.seq_lens_k, case.scale, num_splits=S,
                                           max_seq_len=max_len)
    torch.cuda.synchronize()
    chunks = -(-max_len // 32)
    part_len = -(-chunks // S) * 32
    kp, vp = bits(case.k_pool), bits(case.v_pool)
    bt = case.block_tables.cpu().numpy()
    q = oracle.bf16_bits_to_f64(bits(case.q))
    got_o, got_l = po.cpu().numpy(), pl.cpu().numpy()
    for b, L in enumerate(lens):
        k = oracle.gather_sequence_kv(kp, bt[b], L, 16)
        v = oracle.gather_sequence_kv(vp, bt[b], L, 16)
        bounds = [min(c * part_len, L) for c in range(S)] + [L]
        for h in range(28):
            oc, lc = oracle.split_partials_ref(q[b, h], k[:, h // 7], v[:, h // 7], case.scale,
                                               L, bounds)
            r = b * 28 + h
            assert_parity(got_o[r], oc, f"partials b={b} h={h}", max_abs=2e-3, mean_abs=2e-4)
            assert_lse(got_l[r], lc, f"partial lse b={b} h={h}")
    out_r, lse_r = pa.paged_attn_splitk_reduce(po, pl)
    out_d, lse_d = pa.paged_attn_decode(case.q, case.k_pool, case.v_pool, case.block_tables,
                                        case.seq_lens_k, case.scale, max_seq_len=max_len,
                                        num_splits=S, return_lse=True)
    torch.cuda.synchronize()
    if S > 1:
        assert np.array_equal(bits(out_r.view(case.B, 28, 128)), bits(out_d))
        assert np.array_equal(lse_r.view(case.B, 28).cpu().numpy(), lse_d.cpu().numpy())
