"""FP8 E4M3 pools with one scale per (page, KV head) (reading F2'): the quantising
page write bit-exact against the oracle, decode and prefill against the oracle's
attention over the pools dequantised page by page."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_flashattention_amd as pa
from oracle import fp8 as of
from tests.parity import as_f64, assert_lse, assert_parity, pools_after_write
from workloads import bits, document_ranges, make_case, random_e4m3_codes

pytestmark = pytest.mark.gpu


def page_amax_scales(pool_bits):
    """Per-(page, KV head) scales at amax / 448 over each page's finite values (the
    generator's poison left out; pages without data get scale 1)."""
    x = oracle.bf16_bits_to_f64(pool_bits)
    ok = np.isfinite(x) & (np.abs(x) < 1e4)
    a = np.where(ok, np.abs(x), 0.0).max(axis=(1, 3))          # [P, Hkv]
    return np.where(a > 0, a / 448.0, 1.0).astype(np.float32)


def _codes_and_scales(case, kp_bits, vp_bits):
    ks, vs = page_amax_scales(kp_bits), page_amax_scales(vp_bits)
    return of.quantize_ref(kp_bits, of.page_scales(ks)), of.quantize_ref(vp_bits, of.page_scales(vs)), ks, vs


def _dev(x):
    return torch.as_tensor(np.ascontiguousarray(x), device="cuda")


def test_page_scaled_write_is_bit_exact(require_gpu):
    case = make_case("w8p", hist_lens=[20, 0, 33, 70], q_lens=[5, 40, 1, 130], write_new=True,
                     Hq=8, Hkv=2, D=128, page_size=16, seed=21, device="cuda")
    P = case.k_pool.shape[0]
    rng = np.random.default_rng(22)
    ks = (2.0 ** rng.uniform(-9, 1, (P, 2))).astype(np.float32)
    vs = (2.0 ** rng.uniform(-9, 1, (P, 2))).astype(np.float32)
    k0 = random_e4m3_codes(tuple(case.k_pool.shape), 23, "cuda")
    v0 = random_e4m3_codes(tuple(case.k_pool.shape), 24, "cuda")
    kr, vr = of.kv_write_fp8_ref(k0.cpu().numpy(), v0.cpu().numpy(), bits(case.k_new),
                                 bits(case.v_new), case.cu_new.cpu().numpy(),
                                 case.start_pos.cpu().numpy(), case.block_tables.cpu().numpy(), 16,
                                 ks, vs)
    pa.kv_page_write_fp8(k0, v0, case.k_new, case.v_new, case.cu_new, case.start_pos,
                         case.block_tables, _dev(ks), _dev(vs), validate=True)
    torch.cuda.synchronize()
    assert "scales per page" in pa.describe_launch()
    assert np.array_equal(k0.cpu().numpy(), kr)
    assert np.array_equal(v0.cpu().numpy(), vr)


DECODE = [
    # lens, Hq, Hkv, D, ps, splits, window, alibi
    ([3000, 17, 999, 4096], 28, 4, 128, 16, 0, 0, False),
    ([1, 15, 16, 17, 500], 8, 2, 128, 16, 3, 0, False),
    ([200, 1000], 16, 1, 128, 64, 5, 0, False),
    ([513, 77, 1], 7, 1, 64, 32, 0, 0, False),
    ([2000, 3000], 28, 4, 128, 16, 2, 300, True),
    ([(37 * i) % 701 for i in range(64)], 16, 8, 128, 16, 1, 0, False),   # one-wave grid
]


@pytest.mark.parametrize("lens,Hq,Hkv,D,ps,splits,window,alibi", DECODE)
def test_decode_page_scales(require_gpu, lens, Hq, Hkv, D, ps, splits, window, alibi):
    print(f"[fp8 pages decode] lens={lens[:6]} Hq={Hq} Hkv={Hkv} D={D} ps={ps} S={splits} "
          f"w={window} alibi={alibi}", flush=True)
    case = make_case("dp8", seq_lens=lens, Hq=Hq, Hkv=Hkv, D=D, page_size=ps, seed=sum(lens) + ps,
                     device="cuda", window=window,
                     num_pages=sum(-(-L // ps) for L in lens) + 3)
    kc, vc, ks, vs = _codes_and_scales(case, bits(case.k_pool), bits(case.v_pool))
    slopes = None
    if alibi:
        slopes = torch.tensor([2.0 ** (-(h + 1) / 3) for h in range(Hq)], dtype=torch.float32,
                              device="cuda")
    out, lse = pa.paged_attn_decode_fp8(case.q, _dev(kc), _dev(vc), case.block_tables,
                                        case.seq_lens_k, case.scale, _dev(ks), _dev(vs),
                                        max_seq_len=max(lens), num_splits=splits,
                                        return_lse=True, validate=True, window_left=window,
                                        alibi_slopes=slopes)
    torch.cuda.synchronize()
    assert "scales per page" in pa.describe_launch()
    o_ref, l_ref = oracle.attention_ref(
        bits(case.q), of.dequantize_pool(kc, ks), of.dequantize_pool(vc, vs),
        case.block_tables.cpu().numpy(), case.seq_lens_k.cpu().numpy(),
        case.cu_seqlens_q.cpu().numpy(), case.scale, False, ps, window,
        None if slopes is None else slopes.cpu().numpy())
    assert_parity(as_f64(out), o_ref, "decode fp8 page scales")
    assert_lse(as_f64(lse), l_ref, "decode fp8 page scales lse")


PREFILL = [
    # hist, q_lens, Hq, Hkv, D, ps, causal, splits, window, docs
    ([0, 300], [200, 100], 8, 2, 128, 16, True, 1, 0, 0),         # 4 waves
    ([0, 0], [1100, 300], 8, 2, 128, 16, True, 1, 0, 0),          # 8 waves
    ([500, 0], [600, 513], 8, 4, 128, 32, False, 1, 0, 0),        # non-causal, page 32
    ([100, 40], [700, 90], 8, 2, 64, 64, True, 1, 0, 0),          # D 64, page 64
    ([3000, 0], [512, 2500], 8, 2, 128, 16, True, 3, 0, 0),       # key parts + merge
    ([0, 200], [900, 60], 8, 2, 128, 16, True, 1, 150, 3),        # window + documents
]


@pytest.mark.parametrize("hist,ql,Hq,Hkv,D,ps,causal,splits,window,docs", PREFILL)
def test_prefill_page_scales(require_gpu, hist, ql, Hq, Hkv, D, ps, causal, splits, window, docs):
    print(f"[fp8 pages prefill] hist={hist} q={ql} Hq={Hq} Hkv={Hkv} D={D} ps={ps} "
          f"causal={causal} S={splits} w={window} docs={docs}", flush=True)
    case = make_case("pp8", hist_lens=hist, q_lens=ql, write_new=True, causal=causal, Hq=Hq,
                     Hkv=Hkv, D=D, page_size=ps, seed=sum(hist) + sum(ql) + ps, device="cuda",
                     window=window, num_pages=sum(-(-(h + n) // ps) for h, n in zip(hist, ql)) + 2)
    kp, vp = pools_after_write(case)
    kc, vc, ks, vs = _codes_and_scales(case, kp, vp)
    kr = document_ranges(case.seq_lens, case.q_lens, docs, 31) if docs else None
    out, lse = pa.paged_attn_prefill_varlen_fp8(
        case.q, _dev(kc), _dev(vc), case.cu_seqlens_q, case.seq_lens_k, case.block_tables,
        case.scale, _dev(ks), _dev(vs), causal=causal, max_q_len=case.max_q_len,
        num_splits=splits, return_lse=True, validate=True, window_left=window,
        key_ranges=None if kr is None else (_dev(kr[0]), _dev(kr[1])))
    torch.cuda.synchronize()
    desc = pa.describe_launch()
    assert "scales per page" in desc, desc
    o_ref, l_ref = oracle.attention_ref(
        bits(case.q), of.dequantize_pool(kc, ks), of.dequantize_pool(vc, vs),
        case.block_tables.cpu().numpy(), case.seq_lens_k.cpu().numpy(),
        case.cu_seqlens_q.cpu().numpy(), case.scale, causal, ps, window, None, kr)
    assert_parity(as_f64(out), o_ref, "prefill fp8 page scales")
    assert_lse(as_f64(lse), l_ref, "prefill fp8 page scales lse")


def test_write_then_decode_with_page_scales(require_gpu):
    """New tokens quantised into their pages under each page's scales, then decoded:
    the oracle's quantising write and attention over the dequantised pages."""
    case = make_case("wd8", hist_lens=[300, 1000, 31], q_lens=[1, 1, 1], write_new=True,
                     Hq=28, Hkv=4, D=128, page_size=16, seed=41, device="cuda")
    P = case.k_pool.shape[0]
    kc0, vc0, ks, vs = _codes_and_scales(case, bits(case.k_pool), bits(case.v_pool))
    # pages the writer fills start with unrelated codes
    kc0 = np.where(np.isnan(oracle.bf16_bits_to_f64(bits(case.k_pool))), 0x11, kc0).astype(np.uint8)
    vc0 = np.where(np.isnan(oracle.bf16_bits_to_f64(bits(case.v_pool))), 0x11, vc0).astype(np.uint8)
    k8, v8 = _dev(kc0), _dev(vc0)
    pa.kv_page_write_fp8(k8, v8, case.k_new, case.v_new, case.cu_new, case.start_pos,
                         case.block_tables, _dev(ks), _dev(vs))
    out = pa.paged_attn_decode_fp8(case.q, k8, v8, case.block_tables, case.seq_lens_k,
                                   case.scale, _dev(ks), _dev(vs), max_seq_len=1001)
    torch.cuda.synchronize()
    kr, vr = of.kv_write_fp8_ref(kc0, vc0, bits(case.k_new), bits(case.v_new),
                                 case.cu_new.cpu().numpy(), case.start_pos.cpu().numpy(),
                                 case.block_tables.cpu().numpy(), 16, ks, vs)
    assert np.array_equal(k8.cpu().numpy(), kr) and np.array_equal(v8.cpu().numpy(), vr)
    o_ref, _ = oracle.attention_ref(
        bits(case.q), of.dequantize_pool(kr, ks), of.dequantize_pool(vr, vs),
        case.block_tables.cpu().numpy(), case.seq_lens_k.cpu().numpy(),
        case.cu_seqlens_q.cpu().numpy(), case.scale, False, 16)
    assert_parity(as_f64(out), o_ref, "write then decode, page scales")
    assert P > 0


def test_prefill_page_scales_with_alibi_are_refused(require_gpu):
    case = make_case("ra8", hist_lens=[0], q_lens=[64], write_new=True, causal=True, Hq=8, Hkv=2,
                     D=128, page_size=16, seed=5, device="cuda")
    P = case.k_pool.shape[0]
    k8 = torch.zeros(tuple(case.k_pool.shape), dtype=torch.uint8, device="cuda")
    sc = torch.ones((P, 2), dtype=torch.float32, device="cuda")
    slopes = torch.ones(8, dtype=torch.float32, device="cuda")
    with pytest.raises(pa.PagedAttnError, match="UNSUPPORTED"):
        pa.paged_attn_prefill_varlen_fp8(case.q, k8, k8, case.cu_seqlens_q, case.seq_lens_k,
                                         case.block_tables, case.scale, sc, sc, causal=True,
                                         max_q_len=64, alibi_slopes=slopes)


def _spread_scales(P, Hkv, seed, lo, hi):
    """Scales 2^u per (page, KV head), u uniform in [lo, hi]: neighbouring pages differ
    by up to 2^(hi - lo), so a scale taken from the wrong page or head shows."""
    rng = np.random.default_rng(seed)
    return (2.0 ** rng.uniform(lo, hi, (P, Hkv))).astype(np.float32)


@pytest.mark.parametrize("kind", ["decode", "prefill", "prefill_parts"])
def test_scales_spread_over_pages(require_gpu, kind):
    """Random codes under scales spread over 2^4 per page and head (keys) and 2^3
    (values): decode and prefill against the oracle on the same dequantised pages."""
    print(f"[fp8 pages spread] {kind}", flush=True)
    if kind == "decode":
        case = make_case("sp8", seq_lens=[700, 33, 2048, 16], Hq=16, Hkv=4, D=128, page_size=16,
                         seed=61, device="cuda")
    else:
        case = make_case("sp8p", hist_lens=[400, 0], q_lens=[300, 700], write_new=True,
                         causal=True, Hq=8, Hkv=2, D=128, page_size=16, seed=62, device="cuda")
    shape = tuple(case.k_pool.shape)
    P, Hkv = shape[0], shape[2]
    kc, vc = random_e4m3_codes(shape, 63, "cuda"), random_e4m3_codes(shape, 64, "cuda")
    ks, vs = _spread_scales(P, Hkv, 65, -8, -4), _spread_scales(P, Hkv, 66, -6, -3)
    if kind == "decode":
        out, lse = pa.paged_attn_decode_fp8(case.q, kc, vc, case.block_tables, case.seq_lens_k,
                                            case.scale, _dev(ks), _dev(vs), max_seq_len=2048,
                                            num_splits=4, return_lse=True, validate=True)
    else:
        out, lse = pa.paged_attn_prefill_varlen_fp8(
            case.q, kc, vc, case.cu_seqlens_q, case.seq_lens_k, case.block_tables, case.scale,
            _dev(ks), _dev(vs), causal=True, max_q_len=case.max_q_len,
            num_splits=2 if kind == "prefill_parts" else 1, return_lse=True, validate=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_ref(
        bits(case.q), of.dequantize_pool(kc.cpu().numpy(), ks),
        of.dequantize_pool(vc.cpu().numpy(), vs), case.block_tables.cpu().numpy(),
        case.seq_lens_k.cpu().numpy(), case.cu_seqlens_q.cpu().numpy(), case.scale,
        kind != "decode", 16)
    assert_parity(as_f64(out), o_ref, f"{kind} fp8 spread page scales")
    assert_lse(as_f64(lse), l_ref, f"{kind} fp8 spread page scales lse")
