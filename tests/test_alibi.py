"""GPU parity of the ALiBi score bias (alibi_slopes) against the oracle.

The score of query head h at absolute position p against key j gets
slope_h * (j - p) added after the softmax scale.  Checked: decode (bf16 and FP8
pools, with and without a window, several split counts), prefill (causal and not,
128- and 256-row work-groups, with a window, with key parts), both at full size on
sampled rows, and zero slopes giving the plain kernels' bits.
"""

import numpy as np
import pytest
import torch

import paged_kv_flashattention_amd as pa
from oracle import fp8 as of
from tests.parity import (as_f64, assert_lse, assert_parity, oracle_full, oracle_rows,
                          pools_after_write)
from workloads import bits, make_case, make_config

pytestmark = pytest.mark.gpu


def slopes(Hq, scale=1.0):
    """The geometric ALiBi slopes 2^(-8 (h + 1) / Hq), as float32 on the device."""
    s = np.float32(scale) * 2.0 ** (-8.0 * (np.arange(Hq) + 1) / Hq)
    return torch.tensor(s, dtype=torch.float32, device="cuda")


def host(t):
    return t.cpu().numpy().astype(np.float64)


DECODE = [
    # seq_lens, Hq, Hkv, D, ps, splits, window
    ([1, 15, 16, 17, 100], 8, 2, 128, 16, 1, 0),
    ([127, 4096, 33, 64], 28, 4, 128, 16, 0, 0),
    ([127, 4096, 33, 64], 28, 4, 128, 16, 7, 300),
    ([0, 5, 0, 300], 32, 8, 128, 16, 3, 0),
    ([2000, 1000], 16, 1, 64, 64, 4, 0),
    ([(37 * i) % 701 for i in range(64)], 16, 8, 128, 16, 1, 0),
]


@pytest.mark.parametrize("lens,Hq,Hkv,D,ps,splits,window", DECODE)
def test_alibi_decode_parity(require_gpu, lens, Hq, Hkv, D, ps, splits, window):
    print(f"[alibi decode] lens={lens[:6]} Hq={Hq} Hkv={Hkv} D={D} S={splits} w={window}",
          flush=True)
    case = make_case("ad", seq_lens=lens, Hq=Hq, Hkv=Hkv, D=D, page_size=ps,
                     seed=sum(lens) + 3, num_pages=sum(-(-L // ps) for L in lens) + 5,
                     device="cuda", window=window)
    sl = slopes(Hq)
    out, lse = pa.paged_attn_decode(case.q, case.k_pool, case.v_pool, case.block_tables,
                                    case.seq_lens_k, case.scale, max_seq_len=case.max_seq_len,
                                    num_splits=splits, return_lse=True, validate=True,
                                    window_left=window, alibi_slopes=sl)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_full(case, alibi=host(sl))
    assert_parity(as_f64(out), o_ref, "alibi decode")
    assert_lse(as_f64(lse), l_ref, "alibi decode lse")


def test_alibi_fp8_decode_parity(require_gpu):
    case = make_case("ad8", seq_lens=[3000, 45, 1200], Hq=28, Hkv=4, D=128, page_size=16,
                     seed=18, device="cuda")
    ks, vs = 0.011, 0.009
    kc = of.quantize_ref(bits(case.k_pool), ks)
    vc = of.quantize_ref(bits(case.v_pool), vs)
    sl = slopes(28, 0.5)
    out, lse = pa.paged_attn_decode_fp8(case.q, torch.from_numpy(kc).cuda(),
                                        torch.from_numpy(vc).cuda(), case.block_tables,
                                        case.seq_lens_k, case.scale, ks, vs,
                                        max_seq_len=3000, return_lse=True, alibi_slopes=sl)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_full(case, of.dequantize_pool(kc, ks), of.dequantize_pool(vc, vs),
                               alibi=host(sl))
    assert_parity(as_f64(out), o_ref, "alibi fp8 decode")
    assert_lse(as_f64(lse), l_ref, "alibi fp8 decode lse")


def write(case):
    pa.kv_page_write(case.k_pool, case.v_pool, case.k_new, case.v_new, case.cu_new,
                     case.start_pos, case.block_tables, validate=True)


PREFILL = [
    # hist, q_lens, Hq, Hkv, D, ps, causal, window, splits (None: one pass)
    ([0, 0], [127, 300], 8, 2, 128, 16, True, 0, None),
    ([200, 31, 0], [129, 1, 64], 8, 2, 128, 16, True, 0, None),
    ([17, 0], [50, 130], 8, 8, 64, 32, True, 100, None),
    ([300, 0, 7], [40, 129, 1], 8, 2, 128, 16, False, 0, None),
    ([500, 0], [1030, 260], 8, 2, 128, 32, True, 0, None),         # 256-row work-groups
    ([4113, 214], [512, 40], 8, 2, 128, 16, True, 0, 4),           # key parts
]


@pytest.mark.parametrize("hist,ql,Hq,Hkv,D,ps,causal,window,splits", PREFILL)
def test_alibi_prefill_parity(require_gpu, hist, ql, Hq, Hkv, D, ps, causal, window, splits):
    print(f"[alibi prefill] hist={hist} q={ql} Hq={Hq} D={D} causal={causal} w={window} "
          f"S={splits}", flush=True)
    case = make_case("ap", hist_lens=hist, q_lens=ql, write_new=True, causal=causal, Hq=Hq,
                     Hkv=Hkv, D=D, page_size=ps, seed=sum(ql) + 5, device="cuda",
                     num_pages=sum(-(-(h + n) // ps) for h, n in zip(hist, ql)) + 2,
                     window=window)
    kp, vp = pools_after_write(case)
    write(case)
    sl = slopes(Hq)
    kw = dict(causal=causal, max_q_len=case.max_q_len, return_lse=True, validate=True,
              window_left=window, alibi_slopes=sl)
    if splits is None:
        out, lse = pa.paged_attn_prefill_varlen(case.q, case.k_pool, case.v_pool,
                                                case.cu_seqlens_q, case.seq_lens_k,
                                                case.block_tables, case.scale, **kw)
    else:
        out, lse = pa.paged_attn_prefill_varlen_splitk(case.q, case.k_pool, case.v_pool,
                                                       case.cu_seqlens_q, case.seq_lens_k,
                                                       case.block_tables, case.scale,
                                                       num_splits=splits, **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_full(case, kp, vp, alibi=host(sl))
    assert_parity(as_f64(out), o_ref, "alibi prefill")
    assert_lse(as_f64(lse), l_ref, "alibi prefill lse")


def test_zero_slopes_give_the_plain_results(require_gpu):
    """slope 0 adds exactly 0 to every score: decode equals the plain launch bit for
    bit; prefill with ALiBi walks the key tiles downwards, so its softmax reference
    and hence the bf16 rounding of P differ from the plain launch's: the two agree
    within half the parity tolerance."""
    case = make_case("az", hist_lens=[300, 0], q_lens=[70, 129], write_new=True, causal=True,
                     Hq=8, Hkv=2, D=128, page_size=16, seed=6, device="cuda")
    write(case)
    z = torch.zeros(8, dtype=torch.float32, device="cuda")
    args = (case.q, case.k_pool, case.v_pool, case.cu_seqlens_q, case.seq_lens_k,
            case.block_tables, case.scale)
    a, la = pa.paged_attn_prefill_varlen(*args, causal=True, max_q_len=129, return_lse=True)
    b, lb = pa.paged_attn_prefill_varlen(*args, causal=True, max_q_len=129, return_lse=True,
                                         alibi_slopes=z)
    torch.cuda.synchronize()
    assert_parity(as_f64(b), as_f64(a), "zero slopes vs plain", max_abs=1e-2, mean_abs=1e-3)
    la64 = as_f64(la)
    assert (np.abs(la64 - as_f64(lb)) <= 1e-3 * np.maximum(1.0, np.abs(la64))).all()
    d = make_case("azd", seq_lens=[700, 33, 129], Hq=8, Hkv=2, D=128, page_size=16, seed=7,
                  device="cuda")
    dargs = (d.q, d.k_pool, d.v_pool, d.block_tables, d.seq_lens_k, d.scale)
    a, la = pa.paged_attn_decode(*dargs, max_seq_len=700, num_splits=2, return_lse=True)
    b, lb = pa.paged_attn_decode(*dargs, max_seq_len=700, num_splits=2, return_lse=True,
                                 alibi_slopes=z)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


def test_alibi_causal_prefill_full_size_sampled(require_gpu):
    """Dense causal prefill (4 x 4096, Hq 32, Hkv 8) with geometric ALiBi slopes."""
    case = make_config("causal_prefill", "cuda")
    print("[alibi prefill] causal_prefill full size", flush=True)
    kp, vp = pools_after_write(case)
    write(case)
    sl = slopes(32)
    out, lse = pa.paged_attn_prefill_varlen(case.q, case.k_pool, case.v_pool, case.cu_seqlens_q,
                                            case.seq_lens_k, case.block_tables, case.scale,
                                            causal=True, max_q_len=4096, return_lse=True,
                                            alibi_slopes=sl)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    rows = [(int(t), int(h)) for t, h in zip(rng.integers(0, case.T, 40), rng.integers(0, 32, 40))]
    rows += [(0, 0), (4095, 31), (4096, 4), (case.T - 1, 17)]
    o_ref, l_ref = oracle_rows(case, rows, kp, vp, alibi=host(sl))
    got = np.stack([as_f64(out[t, h]) for t, h in rows])
    assert_parity(got, o_ref, "alibi causal_prefill sampled")
    assert_lse(np.array([float(lse[t, h]) for t, h in rows]), l_ref, "alibi prefill lse")


def test_alibi_decode_full_size_sampled(require_gpu):
    """Qwen2.5-7B-shaped decode (32 x 8192) with ALiBi, automatic splits."""
    case = make_config("qwen7b_decode", "cuda")
    sl = slopes(28)
    print("[alibi decode] qwen7b full size", flush=True)
    out, lse = pa.paged_attn_decode(case.q, case.k_pool, case.v_pool, case.block_tables,
                                    case.seq_lens_k, case.scale, max_seq_len=8192,
                                    return_lse=True, alibi_slopes=sl)
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    rows = [(int(b), int(h)) for b in rng.choice(32, 6, replace=False)
            for h in rng.choice(28, 4, replace=False)]
    o_ref, l_ref = oracle_rows(case, rows, alibi=host(sl))
    got = np.stack([as_f64(out[b, h]) for b, h in rows])
    assert_parity(got, o_ref, "alibi qwen7b sampled")
    assert_lse(np.array([float(lse[b, h]) for b, h in rows]), l_ref, "alibi qwen7b lse")
