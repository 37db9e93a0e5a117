"""The mixed step in one launch (paged_attn_mixed): a step's prefill chunks and decode
rows over the same pools, computed by one kernel whose first work-groups run decode
items and the rest prefill items, then the merges.  Every row against the oracle;
bit-identity with the separate entry points where both take the same work-group
shapes."""

import numpy as np
import pytest
import torch

import paged_kv_flashattention_amd as pa
from tests.parity import (as_f64, assert_lse, assert_parity, oracle_by_sequence, oracle_full,
                          pools_after_write)
from workloads import make_case

pytestmark = pytest.mark.gpu


def write(case):
    pa.kv_page_write(case.k_pool, case.v_pool, case.k_new, case.v_new, case.cu_new,
                     case.start_pos, case.block_tables, validate=True)


def parts(case, n_pf):
    """The case's first n_pf sequences as the prefill part, the rest (one query row
    each) as the decode part."""
    cu = case.cu_seqlens_q
    t_pf = int(cu[n_pf])
    assert all(n == 1 for n in case.q_lens[n_pf:])
    pf = (case.q[:t_pf].contiguous(), cu[:n_pf + 1].contiguous(),
          case.seq_lens_k[:n_pf].contiguous(), case.block_tables[:n_pf].contiguous())
    dec = (case.q[t_pf:].contiguous(), case.block_tables[n_pf:].contiguous(),
           case.seq_lens_k[n_pf:].contiguous())
    return pf, dec, t_pf


def run_mixed(case, n_pf, pf_splits, dec_splits, causal=True):
    pf, dec, t_pf = parts(case, n_pf)
    o_p, o_d, l_p, l_d = pa.paged_attn_mixed(
        case.k_pool, case.v_pool, case.scale, prefill=pf if n_pf else None,
        decode=dec if case.B > n_pf else None, causal=causal,
        prefill_max_q_len=max(case.q_lens[:n_pf]) if n_pf else None,
        prefill_num_splits=pf_splits, decode_max_seq_len=max(case.seq_lens[n_pf:], default=0),
        decode_num_splits=dec_splits, return_lse=True, validate=True)
    torch.cuda.synchronize()
    return o_p, o_d, l_p, l_d, t_pf


CASES = [
    # hist, q_lens (prefill runs first, then decode rows), Hq, Hkv, D, ps, causal, S_pf, S_dec
    ([0, 300, 40, 100, 17, 0], [700, 260, 100, 1, 1, 1], 8, 2, 128, 16, True, 1, 1),
    ([2000, 40, 900, 3000, 1, 64, 63], [300, 512, 90, 1, 1, 1, 1], 8, 2, 128, 16, True, 3, 4),
    ([500, 0, 777, 2048], [300, 513, 1, 1], 8, 4, 64, 32, False, 2, 3),
    ([64, 5, 4000, 31], [70, 600, 1, 1], 16, 1, 128, 64, True, 0, 0),
    ([1220, 214, 4113, 82, 3485, 595], [512, 512, 512, 1, 1, 1], 32, 8, 128, 16, True, 2, 2),
    ([100], [1], 28, 4, 128, 16, True, 1, 2),                      # decode only
    ([0, 1500], [1100, 40], 8, 2, 128, 16, True, 0, 1),            # prefill only
]


@pytest.mark.parametrize("hist,ql,Hq,Hkv,D,ps,causal,s_pf,s_dec", CASES)
def test_mixed_matches_oracle(require_gpu, hist, ql, Hq, Hkv, D, ps, causal, s_pf, s_dec):
    n_pf = sum(1 for n in ql if n > 1)
    print(f"[mixed] hist={hist} q={ql} Hq={Hq} Hkv={Hkv} D={D} ps={ps} causal={causal} "
          f"S_pf={s_pf} S_dec={s_dec}", flush=True)
    case = make_case("mx", hist_lens=hist, q_lens=ql, write_new=True, causal=causal, Hq=Hq,
                     Hkv=Hkv, D=D, page_size=ps, seed=sum(hist) + sum(ql) + D, device="cuda")
    kp, vp = pools_after_write(case)
    write(case)
    o_p, o_d, l_p, l_d, t_pf = run_mixed(case, n_pf, s_pf, s_dec, causal)
    desc = pa.describe_launch()
    assert desc.startswith("mixed<"), desc
    # (a decode row, the last position of its sequence, sees every key with or
    # without the causal mask)
    o_ref, l_ref = oracle_full(case, kp, vp)
    if n_pf:
        assert_parity(as_f64(o_p), o_ref[:t_pf], "mixed prefill rows")
        assert_lse(as_f64(l_p), l_ref[:t_pf], "mixed prefill lse")
    else:
        assert o_p is None
    if case.B > n_pf:
        assert_parity(as_f64(o_d), o_ref[t_pf:], "mixed decode rows")
        assert_lse(as_f64(l_d), l_ref[t_pf:], "mixed decode lse")
    else:
        assert o_d is None


def test_mixed_equals_separate_calls(require_gpu):
    """With the same work-group shapes the fused launch computes the same bits as the
    separate entry points: 256-row prefill tiles (max_q_len >= 512) with the same key
    parts, and one-wave decode work-groups (Hkv x splits x B >= 512) with the same
    split count."""
    hist = [3000, 0, 700] + [(97 * i) % 2500 + 1 for i in range(64)]
    ql = [512, 1030, 600] + [1] * 64
    case = make_case("mxs", hist_lens=hist, q_lens=ql, write_new=True, causal=True, Hq=32,
                     Hkv=8, D=128, page_size=16, seed=5, device="cuda")
    write(case)
    o_p, o_d, l_p, l_d, t_pf = run_mixed(case, 3, 3, 1)
    pf, dec, _ = parts(case, 3)
    s_p, s_pl = pa.paged_attn_prefill_varlen_splitk(*pf[:1], case.k_pool, case.v_pool, *pf[1:],
                                                    case.scale, causal=True, max_q_len=1030,
                                                    num_splits=3, return_lse=True)
    s_d, s_dl = pa.paged_attn_decode(dec[0], case.k_pool, case.v_pool, dec[1], dec[2],
                                     case.scale, max_seq_len=max(case.seq_lens[3:]),
                                     num_splits=1, return_lse=True)
    torch.cuda.synchronize()
    assert "W=1" in pa.describe_launch()
    assert torch.equal(o_p, s_p) and torch.equal(l_p, s_pl)
    assert torch.equal(o_d, s_d) and torch.equal(l_d, s_dl)


def test_mixed_rows_without_keys(require_gpu):
    """Decode rows of empty sequences and prefill rows that see no key give O = 0 and
    lse = -inf, next to ordinary rows in the same launch."""
    case = make_case("mxe", hist_lens=[0, 50, 0, 10], q_lens=[600, 300, 1, 1], write_new=True,
                     causal=True, Hq=8, Hkv=2, D=128, page_size=16, seed=9, device="cuda")
    kp, vp = pools_after_write(case)
    write(case)
    pf, dec, t_pf = parts(case, 2)
    lens_p = pf[2].clone()
    lens_p[0] = 0                       # prefill sequence 0: its 600 rows see no key
    lens_d = dec[2].clone()
    lens_d[0] = 0                       # decode sequence 0: empty
    o_p, o_d, l_p, l_d = pa.paged_attn_mixed(
        case.k_pool, case.v_pool, case.scale, prefill=(pf[0], pf[1], lens_p, pf[3]),
        decode=(dec[0], dec[1], lens_d), prefill_max_q_len=600, prefill_num_splits=2,
        decode_max_seq_len=11, decode_num_splits=2, return_lse=True)
    torch.cuda.synchronize()
    assert not o_p[:600].float().abs().sum().item()
    assert bool(torch.all(l_p[:600] == float("-inf")))
    assert not o_d[0].float().abs().sum().item()
    assert bool(torch.all(l_d[0] == float("-inf")))
    o_ref, l_ref = oracle_full(case, kp, vp)
    assert_parity(as_f64(o_p[600:]), o_ref[600:t_pf], "rows after the empty sequence")
    assert_lse(as_f64(l_p[600:]), l_ref[600:t_pf], "rows after the empty sequence lse")
    assert_parity(as_f64(o_d[1:]), o_ref[t_pf + 1:], "decode row after the empty one")


def test_mixed_ragged_step_full_size_one_launch(require_gpu):
    """The full mixed ragged step (five 512-token chunks over their histories, 18
    decode rows; Hq 32 / Hkv 8) with the prefill's planned key parts: every row of both
    parts against the oracle, sequence by sequence."""
    from workloads import make_config
    case = make_config("mixed_ragged", "cuda")
    n_pf = 5
    s_pf = pa.prefill_plan_splits(case.q_lens[:n_pf], case.seq_lens[:n_pf], case.Hq)
    print(f"[mixed] mixed_ragged full size in one launch, S_pf={s_pf}", flush=True)
    kp, vp = pools_after_write(case)
    write(case)
    o_p, o_d, l_p, l_d, _ = run_mixed(case, n_pf, s_pf, 0)
    # the decode part's own split count: the decode's 2 times the 2 waves per item its
    # launch would take
    assert "8 KV heads x 4 splits x 18 rows" in pa.describe_launch(), pa.describe_launch()
    o_ref, l_ref = oracle_by_sequence(case, kp, vp)
    got = np.concatenate([as_f64(o_p), as_f64(o_d)])
    got_l = np.concatenate([as_f64(l_p), as_f64(l_d)])
    assert_parity(got, o_ref, "mixed step in one launch")
    assert_lse(got_l, l_ref, "mixed step in one launch lse")


def test_mixed_workspace_reuse_and_refusals(require_gpu):
    """Two calls in a row on one caller workspace (the second smaller) against the
    oracle; a workspace one byte short is refused before any launch."""
    case = make_case("mxw", hist_lens=[2000, 0, 900, 300], q_lens=[512, 700, 1, 1],
                     write_new=True, causal=True, Hq=8, Hkv=2, D=128, page_size=16, seed=3,
                     device="cuda")
    kp, vp = pools_after_write(case)
    write(case)
    pf, dec, t_pf = parts(case, 2)
    need = pa.mixed_workspace_bytes(8, 2, 128, (2, t_pf, 700, 4), (2, 901, 3))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o_ref, l_ref = oracle_full(case, kp, vp)
    for reps in range(2):
        sub = (pf[0][:512], pf[1][:2], pf[2][:1], pf[3][:1]) if reps else pf
        o_p, o_d = pa.paged_attn_mixed(case.k_pool, case.v_pool, case.scale, prefill=sub,
                                       decode=dec, prefill_num_splits=4, decode_num_splits=3,
                                       workspace=ws)
        torch.cuda.synchronize()
        n = sub[0].shape[0]
        assert_parity(as_f64(o_p), o_ref[:n], f"mixed prefill, call {reps}")
        assert_parity(as_f64(o_d), o_ref[t_pf:], f"mixed decode, call {reps}")
    with pytest.raises(pa.PagedAttnError, match="WORKSPACE"):
        pa.paged_attn_mixed(case.k_pool, case.v_pool, case.scale, prefill=pf, decode=dec,
                            prefill_num_splits=4, decode_num_splits=3, workspace=ws[:need - 1])


@pytest.mark.parametrize("scales,D", [("pool", 128), ("page", 128), ("page", 64)])
def test_mixed_fp8_pools(require_gpu, scales, D):
    """The one-launch step over FP8 E4M3 pools (one scale per pool, or per page and KV
    head): every row against the oracle on the dequantised pools; the prefill rows
    bit-identical to paged_attn_prefill_varlen_fp8 with the same key parts."""
    from oracle import fp8 as of
    from workloads import random_e4m3_codes
    print(f"[mixed fp8] scales={scales} D={D}", flush=True)
    lens = [2500, 700, 3000, 1, 64, 1500]
    ql = [600, 512, 1, 1, 1, 1]
    case = make_case("mx8", seq_lens=lens, q_lens=ql, Hq=16, Hkv=4, D=D, page_size=16,
                     seed=D + len(scales), device="cuda", causal=True)
    shape = tuple(case.k_pool.shape)
    P = shape[0]
    kc, vc = random_e4m3_codes(shape, 31, "cuda"), random_e4m3_codes(shape, 32, "cuda")
    rng = np.random.default_rng(33)
    if scales == "page":
        ks = (2.0 ** rng.uniform(-8, -4, (P, 4))).astype(np.float32)
        vs = (2.0 ** rng.uniform(-6, -3, (P, 4))).astype(np.float32)
        k_arg, v_arg = torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda()
    else:
        ks, vs = 2.0 ** -6, 2.0 ** -4
        k_arg, v_arg = ks, vs
    pf, dec, t_pf = parts(case, 2)
    o_p, o_d, l_p, l_d = pa.paged_attn_mixed(
        kc, vc, case.scale, prefill=pf, decode=dec, prefill_max_q_len=600,
        prefill_num_splits=3, decode_max_seq_len=3000, decode_num_splits=0, return_lse=True,
        validate=True, k_scale=k_arg, v_scale=v_arg)
    torch.cuda.synchronize()
    desc = pa.describe_launch()
    assert "fp8-e4m3" in desc and (("scales per page" in desc) == (scales == "page")), desc
    s_p, s_pl = pa.paged_attn_prefill_varlen_fp8(pf[0], kc, vc, *pf[1:], case.scale, k_arg,
                                                 v_arg, causal=True, max_q_len=600,
                                                 num_splits=3, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o_p, s_p) and torch.equal(l_p, s_pl)
    kd = of.dequantize_pool(kc.cpu().numpy(), ks)
    vd = of.dequantize_pool(vc.cpu().numpy(), vs)
    o_ref, l_ref = oracle_full(case, kd, vd)
    assert_parity(as_f64(o_p), o_ref[:t_pf], "mixed fp8 prefill rows")
    assert_lse(as_f64(l_p), l_ref[:t_pf], "mixed fp8 prefill lse")
    assert_parity(as_f64(o_d), o_ref[t_pf:], "mixed fp8 decode rows")
    assert_lse(as_f64(l_d), l_ref[t_pf:], "mixed fp8 decode lse")
