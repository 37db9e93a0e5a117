"""GPU parity of sliding-window attention (window_left) against the oracle.

A query at absolute position p sees keys j > p - w (and j <= p when causal); a
decode row sits at position seq_len - 1.  Checked: ragged decode and prefill with
windows shorter than a chunk, not a multiple of 32, spanning partitions, and longer
than every sequence; FP8 pools; key-split prefill; window 1, where every row
returns exactly the value row at its own position.
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


def run_decode(case, splits, window, fp8=None):
    args = (case.q,) + ((case.k_pool, case.v_pool) if fp8 is None else fp8[:2])
    rest = (case.block_tables, case.seq_lens_k, case.scale)
    kw = dict(max_seq_len=case.max_seq_len, num_splits=splits, return_lse=True, validate=True,
              window_left=window)
    if fp8 is None:
        out, lse = pa.paged_attn_decode(*args, *rest, **kw)
    else:
        out, lse = pa.paged_attn_decode_fp8(*args, *rest, fp8[2], fp8[3], **kw)
    torch.cuda.synchronize()
    return out, lse


DECODE = [
    # seq_lens, Hq, Hkv, D, ps, splits, window
    ([1, 15, 16, 17, 100], 8, 2, 128, 16, 1, 5),
    ([1, 15, 16, 17, 100], 8, 2, 128, 16, 3, 33),
    ([127, 4096, 33, 64], 28, 4, 128, 16, 0, 1000),
    ([127, 4096, 33, 64], 28, 4, 128, 16, 7, 100),
    ([0, 5, 0, 300], 32, 8, 128, 16, 2, 64),
    ([2000, 1000], 16, 1, 64, 64, 4, 513),
    ([513, 77, 1], 7, 1, 64, 32, 0, 4096),                      # window longer than all
    ([(37 * i) % 701 for i in range(64)], 16, 8, 128, 16, 1, 200),   # one wave per group
]


@pytest.mark.parametrize("lens,Hq,Hkv,D,ps,splits,window", DECODE)
def test_window_decode_parity(require_gpu, lens, Hq, Hkv, D, ps, splits, window):
    print(f"[window decode] lens={lens[:6]} Hq={Hq} Hkv={Hkv} D={D} ps={ps} S={splits} "
          f"w={window}", flush=True)
    case = make_case("wd", seq_lens=lens, Hq=Hq, Hkv=Hkv, D=D, page_size=ps,
                     seed=sum(lens) + window, num_pages=sum(-(-L // ps) for L in lens) + 5,
                     device="cuda", window=window)
    out, lse = run_decode(case, splits, window)
    o_ref, l_ref = oracle_full(case)
    assert_parity(as_f64(out), o_ref, "window decode")
    assert_lse(as_f64(lse), l_ref, "window decode lse")


@pytest.mark.parametrize("splits", [1, 4])
def test_window_one_decode_returns_the_last_value_row_bit_exact(require_gpu, splits):
    lens = [1, 40, 700, 33]
    case = make_case("w1", seq_lens=lens, Hq=8, Hkv=2, D=128, page_size=16, seed=3,
                     device="cuda", window=1)
    out, _ = run_decode(case, splits, 1)
    bt = case.block_tables.cpu().numpy()
    for b, L in enumerate(lens):
        page, slot = int(bt[b][(L - 1) // 16]), (L - 1) % 16
        for h in range(8):
            assert torch.equal(out[b, h].view(torch.int16),
                               case.v_pool[page, slot, h // 4].view(torch.int16))


def test_window_fp8_decode_parity(require_gpu):
    case = make_case("w8", seq_lens=[3000, 45, 1200], Hq=28, Hkv=4, D=128, page_size=16,
                     seed=8, device="cuda", window=700)
    ks, vs = 0.011, 0.009
    kc = of.quantize_ref(bits(case.k_pool), ks)
    vc = of.quantize_ref(bits(case.v_pool), vs)
    fp8 = (torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda(), ks, vs)
    out, lse = run_decode(case, 0, 700, fp8)
    o_ref, l_ref = oracle_full(case, of.dequantize_pool(kc, ks), of.dequantize_pool(vc, vs))
    assert_parity(as_f64(out), o_ref, "window fp8 decode")
    assert_lse(as_f64(lse), l_ref, "window fp8 decode lse")


def write(case):
    pa.kv_page_write(case.k_pool, case.v_pool, case.k_new, case.v_new, case.cu_new,
                     case.start_pos, case.block_tables, validate=True)


PREFILL = [
    # hist, q_lens, Hq, Hkv, D, ps, causal, window, splits (None: one pass)
    ([0, 0], [127, 300], 8, 2, 128, 16, True, 1, None),
    ([200, 31, 0], [129, 1, 64], 8, 2, 128, 16, True, 50, None),
    ([1000, 0], [100, 257], 28, 4, 128, 16, True, 64, None),
    ([17, 0], [50, 130], 8, 8, 64, 32, True, 100, None),
    ([300, 0, 7], [40, 129, 1], 8, 2, 128, 16, False, 77, None),
    ([500, 0], [1030, 260], 8, 2, 128, 32, True, 300, None),     # 256-row work-groups
    ([0], [1100], 4, 2, 64, 16, True, 5000, None),               # window longer than all
    ([4113, 214], [512, 40], 8, 2, 128, 16, True, 2500, 4),      # key parts over the window
    ([3000], [300], 4, 1, 128, 64, False, 1500, 0),
]


@pytest.mark.parametrize("hist,ql,Hq,Hkv,D,ps,causal,window,splits", PREFILL)
def test_window_prefill_parity(require_gpu, hist, ql, Hq, Hkv, D, ps, causal, window, splits):
    print(f"[window prefill] hist={hist} q={ql} Hq={Hq} Hkv={Hkv} D={D} ps={ps} "
          f"causal={causal} w={window} S={splits}", flush=True)
    case = make_case("wp", hist_lens=hist, q_lens=ql, write_new=True, causal=causal, Hq=Hq,
                     Hkv=Hkv, D=D, page_size=ps, seed=sum(ql) + window, device="cuda",
                     num_pages=sum(-(-(h + n) // ps) for h, n in zip(hist, ql)) + 2,
                     window=window)
    kp, vp = pools_after_write(case)
    write(case)
    kw = dict(causal=causal, max_q_len=case.max_q_len, return_lse=True, validate=True,
              window_left=window)
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
    o_ref, l_ref = oracle_full(case, kp, vp)
    assert_parity(as_f64(out), o_ref, "window prefill")
    assert_lse(as_f64(lse), l_ref, "window prefill lse")


def test_window_one_prefill_returns_own_value_rows_bit_exact(require_gpu):
    case = make_case("wp1", hist_lens=[100, 0], q_lens=[70, 300], write_new=True, causal=True,
                     Hq=8, Hkv=2, D=128, page_size=16, seed=4, device="cuda", window=1)
    write(case)
    out = pa.paged_attn_prefill_varlen(case.q, case.k_pool, case.v_pool, case.cu_seqlens_q,
                                       case.seq_lens_k, case.block_tables, case.scale,
                                       causal=True, max_q_len=300, window_left=1)
    torch.cuda.synchronize()
    # the row's own key is the token's new value row
    for h in range(8):
        assert torch.equal(out[:, h].view(torch.int16), case.v_new[:, h // 4].view(torch.int16))


def test_window_decode_full_size_sampled(require_gpu):
    """Qwen2.5-7B-shaped decode (32 x 8192) with a 4,096-key window, automatic splits."""
    case = make_config("qwen7b_decode", "cuda")
    case.window = 4096
    print("[window decode] qwen7b full size, w=4096", flush=True)
    out, lse = run_decode(case, 0, 4096)
    assert "splits=" in pa.describe_launch()
    rng = np.random.default_rng(9)
    rows = [(int(b), int(h)) for b in rng.choice(32, 6, replace=False)
            for h in rng.choice(28, 4, replace=False)]
    o_ref, l_ref = oracle_rows(case, rows)
    got = np.stack([as_f64(out[b, h]) for b, h in rows])
    assert_parity(got, o_ref, "window qwen7b sampled")
    assert_lse(np.array([float(lse[b, h]) for b, h in rows]), l_ref, "window qwen7b lse")


def test_window_causal_prefill_full_size_sampled(require_gpu):
    """Dense causal prefill (4 x 4096, Hq 32, Hkv 8) with a 1,024-key window."""
    case = make_config("causal_prefill", "cuda")
    case.window = 1024
    print("[window prefill] causal_prefill full size, w=1024", flush=True)
    kp, vp = pools_after_write(case)
    write(case)
    out, lse = pa.paged_attn_prefill_varlen(case.q, case.k_pool, case.v_pool, case.cu_seqlens_q,
                                            case.seq_lens_k, case.block_tables, case.scale,
                                            causal=True, max_q_len=4096, return_lse=True,
                                            window_left=1024)
    torch.cuda.synchronize()
    rng = np.random.default_rng(10)
    rows = [(int(t), int(h)) for t, h in zip(rng.integers(0, case.T, 40), rng.integers(0, 32, 40))]
    rows += [(0, 0), (1023, 3), (1024, 4), (4095, 31), (case.T - 1, 17)]
    o_ref, l_ref = oracle_rows(case, rows, kp, vp)
    got = np.stack([as_f64(out[t, h]) for t, h in rows])
    assert_parity(got, o_ref, "window causal_prefill sampled")
    assert_lse(np.array([float(lse[t, h]) for t, h in rows]), l_ref, "window prefill lse")
