"""GPU parity of the FP8 (E4M3) page format.

* kv_page_write_fp8 is bit-exact against the oracle's quantiser and placement,
  including every rounding tie, the subnormal range and the clamp at 448;
* paged_attn_decode_fp8 matches the oracle's attention over the dequantised pools
  (code value times the pool scale) within the bf16 tolerances;
* with unit scales the FP8 decode gives exactly the bf16 decode's bits on pools
  holding the same (bf16-representable) values.
"""

import numpy as np
import pytest
import torch

from oracle import fp8 as of
import paged_kv_flashattention_amd as pa
from tests.parity import (as_f64, assert_lse, assert_parity, oracle_full, oracle_rows,
                          pools_after_write)
from workloads import bits, make_case, make_config, random_e4m3_codes

pytestmark = pytest.mark.gpu


def amax_scale(t: torch.Tensor) -> float:
    """A per-pool scale that maps the largest magnitude of the data to 448 (a
    caller's choice; the library takes any positive finite scale).  The generator's
    poison (NaN pages, +-3e4 past a sequence's end) is left out."""
    x = t.float()
    a = float(x[torch.isfinite(x) & (x.abs() < 1e4)].abs().max())
    return float(np.float32(a / 448.0))


def to_gpu_codes(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes)).cuda()


def write_fp8(case, kp, vp, k_scale, v_scale):
    pa.kv_page_write_fp8(kp, vp, case.k_new, case.v_new, case.cu_new, case.start_pos,
                         case.block_tables, k_scale, v_scale, validate=True)
    torch.cuda.synchronize()


@pytest.mark.parametrize("hist,ql,Hkv,D,ps,scales", [
    ([0, 13, 40], [20, 3, 1], 2, 64, 16, (0.05, 0.02)),
    ([5, 0, 100, 64], [1, 64, 17, 0], 8, 128, 16, (1.0, 3.0)),
    ([31, 0], [70, 1], 1, 128, 32, (0.001, 0.7)),          # most keys clamp at 448
    ([63, 1], [130, 2], 4, 64, 64, (0.0078125, 0.3)),
])
def test_fp8_write_bit_exact(require_gpu, hist, ql, Hkv, D, ps, scales):
    print(f"[fp8 write] hist={hist} q={ql} Hkv={Hkv} D={D} ps={ps} scales={scales}", flush=True)
    case = make_case("w8", hist_lens=hist, q_lens=ql, write_new=True, Hq=Hkv, Hkv=Hkv, D=D,
                     page_size=ps, seed=sum(hist) + D + 8, device="cuda",
                     num_pages=sum(-(-(h + n) // ps) for h, n in zip(hist, ql)) + 3)
    shape = tuple(case.k_pool.shape)
    # start from random codes so that untouched slots are checked too
    kp = random_e4m3_codes(shape, 11, "cuda")
    vp = random_e4m3_codes(shape, 12, "cuda")
    k_ref, v_ref = of.kv_write_fp8_ref(kp.cpu().numpy(), vp.cpu().numpy(), bits(case.k_new),
                                       bits(case.v_new), case.cu_new.cpu().numpy(),
                                       case.start_pos.cpu().numpy(),
                                       case.block_tables.cpu().numpy(), ps, *scales)
    write_fp8(case, kp, vp, *scales)
    assert np.array_equal(kp.cpu().numpy(), k_ref)
    assert np.array_equal(vp.cpu().numpy(), v_ref)


def _edge_values() -> np.ndarray:
    """Every finite E4M3 value, every midpoint between neighbours (a tie), their
    bf16 neighbours (just off a tie), both signs, and magnitudes past 448.  All
    of them are exact bf16 values."""
    pos = of.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    base = np.concatenate([pos, mids, [464.0, 480.0, 1000.0, 32768.0, 2.0 ** -10, 2.0 ** -12]])
    as32 = base.astype(np.float32)
    up = (as32.view(np.uint32) + (1 << 16)).view(np.float32)      # next bf16 up
    down = (np.maximum(as32.view(np.uint32), 1 << 16) - (1 << 16)).view(np.float32)
    vals = np.concatenate([as32, up, down]).astype(np.float64)
    vals = np.concatenate([vals, -vals])
    b = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(((b.astype(np.uint32) << 16).view(np.float32)).astype(np.float64), vals)
    return b


@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 0.5), (3.0, 0.1)])
def test_fp8_write_rounding_edges(require_gpu, k_scale, v_scale):
    """Ties go to the even code and magnitudes past 448 clamp, as the oracle's
    nearest-value encoder says; unit and power-of-two scales put the ties
    exactly on the device's float32 products."""
    vals = _edge_values()
    Hkv, D, ps = 2, 64, 16
    per_tok = Hkv * D
    T = -(-vals.size // per_tok)
    flat = np.zeros(T * per_tok, np.uint16)
    flat[:vals.size] = vals
    k_new = torch.from_numpy(flat.view(np.int16).reshape(T, Hkv, D)).view(torch.bfloat16)
    v_new = torch.from_numpy(flat[::-1].copy().view(np.int16).reshape(T, Hkv, D)).view(
        torch.bfloat16)
    pages = -(-T // ps)
    bt = torch.arange(pages, dtype=torch.int32)[None].flip(1).contiguous()
    cu = torch.tensor([0, T], dtype=torch.int32)
    sp = torch.zeros(1, dtype=torch.int32)
    kp = torch.zeros((pages, ps, Hkv, D), dtype=torch.uint8)
    vp = torch.zeros_like(kp)
    k_ref, v_ref = of.kv_write_fp8_ref(kp.numpy(), vp.numpy(), bits(k_new), bits(v_new),
                                       cu.numpy(), sp.numpy(), bt.numpy(), ps, k_scale, v_scale)
    print(f"[fp8 write] rounding edges: {vals.size} values, scales {k_scale}/{v_scale}", flush=True)
    kg, vg = kp.cuda(), vp.cuda()
    pa.kv_page_write_fp8(kg, vg, k_new.cuda(), v_new.cuda(), cu.cuda(), sp.cuda(), bt.cuda(),
                         k_scale, v_scale)
    torch.cuda.synchronize()
    assert np.array_equal(kg.cpu().numpy(), k_ref)
    assert np.array_equal(vg.cpu().numpy(), v_ref)


def test_fp8_write_full_config(require_gpu):
    """Mixed ragged batch (23 sequences, 2578 new tokens) at its full size."""
    case = make_config("mixed_ragged", "cuda")
    ks, vs = amax_scale(case.k_new), amax_scale(case.v_new)
    shape = tuple(case.k_pool.shape)
    kp = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    vp = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    print(f"[fp8 write] mixed_ragged {case.k_new.shape[0]} tokens", flush=True)
    write_fp8(case, kp, vp, ks, vs)
    zeros = np.zeros(shape, np.uint8)
    k_ref, v_ref = of.kv_write_fp8_ref(zeros, zeros, bits(case.k_new), bits(case.v_new),
                                       case.cu_new.cpu().numpy(), case.start_pos.cpu().numpy(),
                                       case.block_tables.cpu().numpy(), case.page_size, ks, vs)
    assert np.array_equal(kp.cpu().numpy(), k_ref)
    assert np.array_equal(vp.cpu().numpy(), v_ref)


def run_decode_fp8(case, kc, vc, ks, vs, splits, pool_dtype=torch.uint8):
    if pool_dtype != torch.uint8:
        kc, vc = kc.view(pool_dtype), vc.view(pool_dtype)
    out, lse = pa.paged_attn_decode_fp8(case.q, kc, vc, case.block_tables, case.seq_lens_k,
                                        case.scale, ks, vs, max_seq_len=case.max_seq_len,
                                        num_splits=splits, return_lse=True, validate=True)
    torch.cuda.synchronize()
    return out, lse


DECODE = [
    # seq_lens, Hq, Hkv, D, ps, splits
    ([17, 64, 100, 255], 8, 2, 64, 16, 1),
    ([1, 15, 16, 17], 8, 2, 128, 16, 4),
    ([127, 4096, 33, 64], 28, 4, 128, 16, 0),
    ([0, 5, 0, 300], 32, 8, 128, 16, 3),
    ([200, 1000], 16, 1, 128, 64, 5),
    ([513, 77, 1], 7, 1, 64, 64, 0),
    # FP8 pools take one wave per work-group from 1024 work-groups, two from 512
    ([(37 * i) % 701 for i in range(64)], 16, 8, 128, 16, 1),     # 512: two waves
    ([(37 * i) % 701 for i in range(64)], 16, 8, 128, 16, 2),     # 1024: one wave
    ([(53 * i) % 509 for i in range(64)], 8, 8, 64, 16, 2),       # 1024: one wave, D 64
]


@pytest.mark.parametrize("lens,Hq,Hkv,D,ps,splits", DECODE)
def test_fp8_decode_parity(require_gpu, lens, Hq, Hkv, D, ps, splits):
    print(f"[fp8 decode] lens={lens} Hq={Hq} Hkv={Hkv} D={D} ps={ps} S={splits}", flush=True)
    case = make_case("d8", seq_lens=lens, Hq=Hq, Hkv=Hkv, D=D, page_size=ps,
                     seed=sum(lens) + D + 8, num_pages=sum(-(-L // ps) for L in lens) + 5,
                     device="cuda")
    ks, vs = amax_scale(case.k_pool), amax_scale(case.v_pool)
    kc = of.quantize_ref(bits(case.k_pool), ks)
    vc = of.quantize_ref(bits(case.v_pool), vs)
    out, lse = run_decode_fp8(case, to_gpu_codes(kc), to_gpu_codes(vc), ks, vs, splits)
    o_ref, l_ref = oracle_full(case, of.dequantize_pool(kc, ks), of.dequantize_pool(vc, vs))
    assert_parity(as_f64(out), o_ref, "fp8 decode")
    assert_lse(as_f64(lse), l_ref, "fp8 decode lse")
    for b, L in enumerate(lens):
        if L == 0:
            assert (as_f64(out[b]) == 0).all()
            assert np.isneginf(as_f64(lse[b])).all()


def test_fp8_decode_accepts_float8_dtype(require_gpu):
    case = make_case("d8t", seq_lens=[300, 41], Hq=8, Hkv=2, D=128, page_size=16, seed=4,
                     device="cuda")
    ks, vs = 0.01, 0.004
    kc = to_gpu_codes(of.quantize_ref(bits(case.k_pool), ks))
    vc = to_gpu_codes(of.quantize_ref(bits(case.v_pool), vs))
    print("[fp8 decode] uint8 vs float8_e4m3fn pools", flush=True)
    a, la = run_decode_fp8(case, kc, vc, ks, vs, 2)
    b, lb = run_decode_fp8(case, kc, vc, ks, vs, 2, torch.float8_e4m3fn)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(la, lb)


@pytest.mark.parametrize("splits", [1, 3])
def test_unit_scale_fp8_decode_equals_bf16_decode_bitwise(require_gpu, splits):
    """With k_scale = v_scale = 1 the codes widen exactly to the bf16 values a bf16
    pool would hold, and the two paths share every later step."""
    case = make_case("d8u", seq_lens=[700, 33, 129], Hq=28, Hkv=4, D=128, page_size=16,
                     seed=9, device="cuda")
    shape = tuple(case.k_pool.shape)
    kc = random_e4m3_codes(shape, 21, "cuda", 2, 8)
    vc = random_e4m3_codes(shape, 22, "cuda", 2, 8)
    as_bf16 = lambda c: torch.from_numpy(                                       # noqa: E731
        of.e4m3_decode(c.cpu().numpy()).astype(np.float32)).to(torch.bfloat16).cuda()
    kb, vb = as_bf16(kc), as_bf16(vc)
    assert torch.equal(kb.float().cpu().double(),
                       torch.from_numpy(of.e4m3_decode(kc.cpu().numpy())))   # exact widening
    print(f"[fp8 decode] unit scales vs bf16, S={splits}", flush=True)
    o8, l8 = run_decode_fp8(case, kc, vc, 1.0, 1.0, splits)
    o16, l16 = pa.paged_attn_decode(case.q, kb, vb, case.block_tables, case.seq_lens_k,
                                    case.scale, max_seq_len=case.max_seq_len,
                                    num_splits=splits, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o8.view(torch.int16), o16.view(torch.int16))
    assert torch.equal(l8, l16)


def test_fp8_decode_full_size_sampled(require_gpu):
    """Qwen2.5-7B-shaped decode (32 x 8192 keys, Hq 28, Hkv 4, D 128, page 16) over FP8
    pools of seeded random codes, in the benchmark's launch configuration (automatic
    split count); oracle on sampled (sequence, head) rows, dequantising only the
    sampled sequences' pages."""
    case = make_config("qwen7b_decode", "cuda")
    shape = tuple(case.k_pool.shape)
    case.k_pool = case.v_pool = None
    kc = random_e4m3_codes(shape, 1001 * 8 + 1, "cuda")
    vc = random_e4m3_codes(shape, 1001 * 8 + 2, "cuda")
    ks, vs = 0.02, 0.05
    print("[fp8 decode] qwen7b full size", flush=True)
    out, lse = run_decode_fp8(case, kc, vc, ks, vs, 0)
    rng = np.random.default_rng(3)
    rows = [(int(b), int(h)) for b in rng.choice(case.B, 6, replace=False)
            for h in rng.choice(case.Hq, 4, replace=False)]
    bt = case.block_tables.cpu().numpy()
    n = case.max_seq_len // case.page_size
    kd = np.zeros(shape)
    vd = np.zeros(shape)
    for b in sorted({b for b, _ in rows}):
        pages = bt[b, :n].astype(np.int64)
        idx = torch.as_tensor(pages, device="cuda")
        kd[pages] = of.dequantize_pool(kc[idx].cpu().numpy(), ks)
        vd[pages] = of.dequantize_pool(vc[idx].cpu().numpy(), vs)
    o_ref, l_ref = oracle_rows(case, rows, kd, vd)
    got = np.stack([as_f64(out[b, h]) for b, h in rows])
    assert_parity(got, o_ref, "fp8 qwen7b sampled")
    assert_lse(np.array([float(lse[b, h]) for b, h in rows]), l_ref, "fp8 qwen7b lse")
    assert torch.isfinite(out.float()).all()


def test_fp8_write_then_decode_round_trip(require_gpu):
    """The quantising write feeds the FP8 decode: write a ragged batch of new tokens
    into FP8 pools on the device, decode the last token of each sequence, and
    compare with the oracle's attention over its own quantised write."""
    case = make_case("wd8", hist_lens=[0, 0, 0], q_lens=[37, 300, 1], write_new=True, Hq=16,
                     Hkv=4, D=128, page_size=16, seed=77, device="cuda")
    ks, vs = amax_scale(case.k_new), amax_scale(case.v_new)
    shape = tuple(case.k_pool.shape)
    kp = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    vp = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    write_fp8(case, kp, vp, ks, vs)
    lens = case.seq_lens_k
    last = (case.cu_seqlens_q[1:] - 1).long()
    q = case.q[last].contiguous()
    print("[fp8 decode] write then decode", flush=True)
    out, lse = pa.paged_attn_decode_fp8(q, kp, vp, case.block_tables, lens, case.scale, ks, vs,
                                        max_seq_len=300, num_splits=2, return_lse=True)
    torch.cuda.synchronize()
    zeros = np.zeros(shape, np.uint8)
    k_ref, v_ref = of.kv_write_fp8_ref(zeros, zeros, bits(case.k_new), bits(case.v_new),
                                       case.cu_new.cpu().numpy(), case.start_pos.cpu().numpy(),
                                       case.block_tables.cpu().numpy(), 16, ks, vs)
    dcase = make_case("wd8q", seq_lens=[37, 300, 1], Hq=16, Hkv=4, D=128, page_size=16,
                      seed=77, num_pages=shape[0])
    dcase.q = q.cpu()
    dcase.block_tables = case.block_tables.cpu()
    o_ref, l_ref = oracle_full(dcase, of.dequantize_pool(k_ref, ks), of.dequantize_pool(v_ref, vs))
    assert_parity(as_f64(out), o_ref, "fp8 write+decode")
    assert_lse(as_f64(lse), l_ref, "fp8 write+decode lse")


# ---------------------------------------------------------------------------
# prefill over FP8 pools
# ---------------------------------------------------------------------------

def _pool_codes(case, kp_bits, vp_bits):
    """E4M3 codes of the case's pools (after its page write) at amax/448 scales."""
    kx = torch.from_numpy(kp_bits.view(np.int16)).view(torch.bfloat16)
    vx = torch.from_numpy(vp_bits.view(np.int16)).view(torch.bfloat16)
    ks, vs = amax_scale(kx), amax_scale(vx)
    return of.quantize_ref(kp_bits, ks), of.quantize_ref(vp_bits, vs), ks, vs


PREFILL = [
    # hist, q_lens, Hq, Hkv, D, ps, causal, splits, window, alibi
    ([0, 0], [127, 300], 8, 2, 128, 16, True, 1, 0, False),
    ([200, 31, 0], [129, 1, 64], 8, 2, 128, 16, True, 1, 0, False),
    ([17, 0], [50, 130], 8, 8, 64, 32, True, 1, 0, False),          # D 64, 4 waves
    ([0, 0], [1100, 300], 4, 2, 64, 16, True, 1, 0, False),         # D 64, 8 waves
    ([500, 0], [1030, 260], 8, 2, 128, 64, True, 1, 0, False),      # D 128, 8 waves
    ([300, 0, 7], [40, 129, 1], 8, 2, 128, 16, False, 1, 0, False),
    ([1000, 0], [100, 257], 28, 4, 128, 16, True, 1, 200, True),    # window and ALiBi
    ([1000, 0], [100, 257], 28, 4, 128, 16, True, 1, 200, False),   # window only, 4 waves
    ([0, 300], [1100, 70], 8, 2, 128, 16, True, 1, 333, False),     # window only, 8 waves
    ([600, 0], [90, 140], 8, 2, 64, 16, True, 1, 0, True),          # ALiBi only, D 64
    ([2100, 37], [1030, 5], 8, 2, 128, 32, True, 2, 0, True),       # ALiBi, 8 waves, 2 parts
    ([4113, 214], [512, 40], 8, 2, 128, 16, True, 4, 0, False),     # key parts
]


@pytest.mark.parametrize("hist,ql,Hq,Hkv,D,ps,causal,splits,window,alibi", PREFILL)
def test_fp8_prefill_parity(require_gpu, hist, ql, Hq, Hkv, D, ps, causal, splits, window,
                            alibi):
    print(f"[fp8 prefill] hist={hist} q={ql} Hq={Hq} Hkv={Hkv} D={D} ps={ps} causal={causal} "
          f"S={splits} w={window} alibi={alibi}", flush=True)
    case = make_case("p8", hist_lens=hist, q_lens=ql, write_new=True, causal=causal, Hq=Hq,
                     Hkv=Hkv, D=D, page_size=ps, seed=sum(ql) + D + 88, device="cuda",
                     num_pages=sum(-(-(h + n) // ps) for h, n in zip(hist, ql)) + 2,
                     window=window)
    kp, vp = pools_after_write(case)
    kc, vc, ks, vs = _pool_codes(case, kp, vp)
    sl = (torch.tensor(2.0 ** (-8.0 * (np.arange(Hq) + 1) / Hq), dtype=torch.float32,
                       device="cuda") if alibi else None)
    out, lse = pa.paged_attn_prefill_varlen_fp8(
        case.q, to_gpu_codes(kc), to_gpu_codes(vc), case.cu_seqlens_q, case.seq_lens_k,
        case.block_tables, case.scale, ks, vs, causal=causal, max_q_len=case.max_q_len,
        num_splits=splits, return_lse=True, validate=True, window_left=window,
        alibi_slopes=sl)
    torch.cuda.synchronize()
    assert "fp8" in pa.describe_launch()
    o_ref, l_ref = oracle_full(case, of.dequantize_pool(kc, ks), of.dequantize_pool(vc, vs),
                               alibi=None if sl is None else sl.cpu().numpy().astype(np.float64))
    assert_parity(as_f64(out), o_ref, "fp8 prefill")
    assert_lse(as_f64(lse), l_ref, "fp8 prefill lse")


@pytest.mark.parametrize("q_lens", [[129, 300], [1100, 64]])
def test_unit_scale_fp8_prefill_equals_bf16_prefill_bitwise(require_gpu, q_lens):
    """Unit scales: the widened codes are the bf16 values a bf16 pool would hold, and
    both paths run the same kernel body from there."""
    case = make_case("p8u", seq_lens=[300 + q_lens[0], q_lens[1]], q_lens=q_lens, causal=True,
                     Hq=8, Hkv=2, D=128, page_size=16, seed=19, device="cuda")
    shape = tuple(case.k_pool.shape)
    kc = random_e4m3_codes(shape, 31, "cuda", 2, 8)
    vc = random_e4m3_codes(shape, 32, "cuda", 2, 8)
    as_bf16 = lambda c: torch.from_numpy(                                       # noqa: E731
        of.e4m3_decode(c.cpu().numpy()).astype(np.float32)).to(torch.bfloat16).cuda()
    args = (case.q,)
    rest = (case.cu_seqlens_q, case.seq_lens_k, case.block_tables, case.scale)
    o8, l8 = pa.paged_attn_prefill_varlen_fp8(*args, kc, vc, *rest, 1.0, 1.0, causal=True,
                                              max_q_len=max(q_lens), return_lse=True)
    o16, l16 = pa.paged_attn_prefill_varlen(*args, as_bf16(kc), as_bf16(vc), *rest, causal=True,
                                            max_q_len=max(q_lens), return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o8.view(torch.int16), o16.view(torch.int16))
    assert torch.equal(l8, l16)


def test_fp8_causal_prefill_full_size_sampled(require_gpu):
    """Dense causal prefill (4 x 4096, Hq 32, Hkv 8) over FP8 pools of seeded random codes;
    the oracle dequantises only the pages the sampled rows need."""
    case = make_config("causal_prefill", "cuda")
    shape = tuple(case.k_pool.shape)
    case.k_pool = case.v_pool = None
    kc = random_e4m3_codes(shape, 1003 * 8 + 1, "cuda")
    vc = random_e4m3_codes(shape, 1003 * 8 + 2, "cuda")
    ks, vs = 0.02, 0.05
    print("[fp8 prefill] causal_prefill full size", flush=True)
    out, lse = pa.paged_attn_prefill_varlen_fp8(case.q, kc, vc, case.cu_seqlens_q,
                                                case.seq_lens_k, case.block_tables, case.scale,
                                                ks, vs, causal=True, max_q_len=4096,
                                                return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(14)
    rows = [(int(t), int(h)) for t, h in zip(rng.integers(0, case.T, 32), rng.integers(0, 32, 32))]
    rows += [(0, 0), (4095, 31), (case.T - 1, 17)]
    bt = case.block_tables.cpu().numpy()
    kd = np.zeros(shape)
    vd = np.zeros(shape)
    for b in sorted({t // 4096 for t, _ in rows}):
        pages = bt[b, :256].astype(np.int64)
        idx = torch.as_tensor(pages, device="cuda")
        kd[pages] = of.dequantize_pool(kc[idx].cpu().numpy(), ks)
        vd[pages] = of.dequantize_pool(vc[idx].cpu().numpy(), vs)
    o_ref, l_ref = oracle_rows(case, rows, kd, vd)
    got = np.stack([as_f64(out[t, h]) for t, h in rows])
    assert_parity(got, o_ref, "fp8 causal_prefill sampled")
    assert_lse(np.array([float(lse[t, h]) for t, h in rows]), l_ref, "fp8 prefill lse")
    assert torch.isfinite(out.float()).all()


def test_fp8_write_then_prefill_round_trip(require_gpu):
    """The quantising page write feeds the FP8 prefill: a ragged batch of chunks over
    their history, all in FP8 pools."""
    case = make_case("wp8", hist_lens=[0, 0, 0], q_lens=[37, 300, 129], write_new=True,
                     causal=True, Hq=16, Hkv=4, D=128, page_size=16, seed=78, device="cuda")
    ks, vs = amax_scale(case.k_new), amax_scale(case.v_new)
    shape = tuple(case.k_pool.shape)
    kp = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    vp = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    write_fp8(case, kp, vp, ks, vs)
    print("[fp8 prefill] write then prefill", flush=True)
    out, lse = pa.paged_attn_prefill_varlen_fp8(case.q, kp, vp, case.cu_seqlens_q,
                                                case.seq_lens_k, case.block_tables, case.scale,
                                                ks, vs, causal=True, max_q_len=300,
                                                return_lse=True)
    torch.cuda.synchronize()
    zeros = np.zeros(shape, np.uint8)
    k_ref, v_ref = of.kv_write_fp8_ref(zeros, zeros, bits(case.k_new), bits(case.v_new),
                                       case.cu_new.cpu().numpy(), case.start_pos.cpu().numpy(),
                                       case.block_tables.cpu().numpy(), 16, ks, vs)
    o_ref, l_ref = oracle_full(case, of.dequantize_pool(k_ref, ks), of.dequantize_pool(v_ref, vs))
    assert_parity(as_f64(out), o_ref, "fp8 write+prefill")
    assert_lse(as_f64(lse), l_ref, "fp8 write+prefill lse")
