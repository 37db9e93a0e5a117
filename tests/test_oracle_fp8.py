"""Pins for the FP8 (E4M3) part of the oracle, against things other than itself:

* the values the OCP E4M3 format fixes (largest finite 448, smallest normal 2^-6,
  smallest subnormal 2^-9, 1.0, NaN codes);
* a library routine: torch's float8_e4m3fn dtype (decoding every code, and its
  round-to-nearest-even cast for magnitudes up to 448);
* brute force: a pure-Python nearest-value search with ties to even;
* invariants: encode(decode(c)) == c, monotonicity, the quantised page write
  equals the quantised values placed by the bf16 page write;
* planted mistakes (wrong bias, ties away from zero, inverted scale) that must fail.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import fp8 as of
from workloads import bits, make_case


def test_values_the_format_fixes():
    d = of.e4m3_decode(np.array([0x7E, 0x08, 0x01, 0x38, 0xB8, 0x40, 0x00, 0x80], np.uint8))
    assert list(d[:6]) == [448.0, 2.0 ** -6, 2.0 ** -9, 1.0, -1.0, 2.0]
    assert d[6] == 0.0 and d[7] == 0.0 and math.copysign(1.0, d[7]) == -1.0
    nan = of.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))
    assert np.isnan(nan).all()


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = of.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert (both_nan | (ours == ref)).all()
    assert both_nan.sum() == 2


def _brute_encode(x):
    """Nearest finite E4M3 value by a linear scan, ties to the even code."""
    best = None
    for c in range(0x7F):
        v = float(of.e4m3_decode(np.array([c], np.uint8))[0])
        d = abs(abs(x) - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    c = best[1]
    return (c | 0x80) if math.copysign(1.0, x) < 0 else c


def test_encode_matches_brute_force_and_torch():
    rng = np.random.default_rng(7)
    vals = list(of.e4m3_decode(np.arange(0x7F, dtype=np.uint8)))
    mids = [(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]          # every tie
    x = np.array(vals + mids + list(rng.uniform(-448, 448, 400)) +
                 list(rng.normal(0, 0.01, 200)) + [-0.0, -2.0 ** -11, 447.9, -448.0])
    ours = of.e4m3_encode(x)
    brute = np.array([_brute_encode(float(v)) for v in x], np.uint8)
    assert np.array_equal(ours, brute)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(ours, ref.numpy())


def test_round_trip_and_order():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(of.e4m3_encode(of.e4m3_decode(codes)), codes)
    pos = of.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert (np.diff(pos) > 0).all()


def test_quantizer_clamps_and_scales():
    x = np.array([1000.0, -1000.0, 3.0, 0.0], np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)           # exact in bf16
    q = of.quantize_ref(xb, 2.0)
    assert list(of.e4m3_decode(q)) == [448.0, -448.0, 1.5, 0.0]


def test_fp8_page_write_equals_quantised_bf16_write():
    case = make_case("w8", hist_lens=[20, 0, 33], q_lens=[5, 40, 1], write_new=True, Hq=4, Hkv=2,
                     D=64, page_size=16, seed=3)
    kz = np.zeros(case.k_pool.shape, np.uint8)
    vz = np.zeros(case.v_pool.shape, np.uint8)
    kp8, vp8 = of.kv_write_fp8_ref(kz, vz, bits(case.k_new), bits(case.v_new), case.cu_new.numpy(),
                                   case.start_pos.numpy(), case.block_tables.numpy(), 16, 0.05, 0.02)
    kq = of.quantize_ref(bits(case.k_new), 0.05)
    zeros16 = np.zeros(case.k_pool.shape, np.uint16)
    # the same placement as the bf16 writer, applied to the codes
    kp16, _ = oa.kv_write_ref(zeros16, zeros16, kq.astype(np.uint16), kq.astype(np.uint16),
                              case.cu_new.numpy(), case.start_pos.numpy(),
                              case.block_tables.numpy(), 16)
    assert np.array_equal(kp8.astype(np.uint16), kp16)
    assert vp8.any()


@pytest.mark.parametrize("mutant", ["bias8", "ties_away", "scale_inverted"])
def test_planted_fp8_mistakes_are_caught(monkeypatch, mutant):
    if mutant == "bias8":
        real = of.e4m3_decode
        monkeypatch.setattr(of, "e4m3_decode", lambda c: real(c) * 0.5)
        with pytest.raises(AssertionError):
            test_values_the_format_fixes()
    elif mutant == "ties_away":
        real = of.e4m3_encode
        ties = np.array([(a + b) / 2 for a, b in zip(of._POS_VALUES[:-1], of._POS_VALUES[1:])])

        def away(x):
            x = np.asarray(x, np.float64)
            up = real(np.minimum(np.nextafter(np.abs(x), np.inf), of.E4M3_MAX) * np.sign(x))
            return np.where(np.isin(np.abs(x), ties), up, real(x)).astype(np.uint8)
        monkeypatch.setattr(of, "e4m3_encode", away)
        with pytest.raises(AssertionError):
            test_encode_matches_brute_force_and_torch()
    else:
        real_q = of.quantize_ref
        monkeypatch.setattr(of, "quantize_ref", lambda x, scale: real_q(x, 1.0 / scale))
        with pytest.raises(AssertionError):
            test_quantizer_clamps_and_scales()


# ----------------------------------------------------------------------------
# per-(page, KV head) scales (F2')
# ----------------------------------------------------------------------------

def _page_scales(P, Hkv, seed):
    rng = np.random.default_rng(seed)
    return (2.0 ** rng.uniform(-8, 2, size=(P, Hkv))).astype(np.float32)


def test_page_scales_all_equal_are_the_pool_scale():
    rng = np.random.default_rng(12)
    x = rng.normal(0, 3, size=(6, 16, 2, 64)).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    ks = np.full((6, 2), 0.0375, np.float32)
    assert np.array_equal(of.quantize_ref(xb, of.page_scales(ks)), of.quantize_ref(xb, 0.0375))
    c = of.quantize_ref(xb, 0.0375)
    assert np.array_equal(of.dequantize_pool(c, ks), of.dequantize_pool(c, 0.0375))


def test_page_scales_match_brute_force_per_element():
    """Every element is encoded by the brute-force scan of y = x * fl32(1 / s) for
    the scale of its own (page, head)."""
    rng = np.random.default_rng(13)
    x = rng.normal(0, 2, size=(3, 4, 2, 8)).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    xf = oa.bf16_bits_to_f64(xb)
    ks = _page_scales(3, 2, 14)
    codes = of.quantize_ref(xb, of.page_scales(ks))
    for p in range(3):
        for h in range(2):
            inv = np.float32(1.0) / ks[p, h]
            for r in range(4):
                for d in range(8):
                    y = float(np.clip(np.float32(xf[p, r, h, d]) * inv, -448.0, 448.0))
                    assert codes[p, r, h, d] == _brute_encode(y), (p, h, r, d)
    # dequantisation multiplies each code by its own page's scale
    deq = of.dequantize_pool(codes, ks)
    assert np.array_equal(deq[2, :, 1], of.e4m3_decode(codes[2, :, 1]) * float(ks[2, 1]))
    # and stays within half an E4M3 step (relative 2^-4) of the value, away from clamping
    ok = np.abs(xf) < 448.0 * ks[:, None, :, None] * 0.9
    rel = np.abs(deq - xf) / np.maximum(np.abs(xf), 2.0 ** -6 * ks[:, None, :, None])
    assert (rel[ok] <= 2.0 ** -4 + 1e-12).all()


def test_page_scaled_write_uses_each_pages_scale():
    case = make_case("w8p", hist_lens=[20, 0, 33], q_lens=[5, 40, 1], write_new=True, Hq=4,
                     Hkv=2, D=64, page_size=16, seed=4)
    P = case.k_pool.shape[0]
    ks, vs = _page_scales(P, 2, 15), _page_scales(P, 2, 16)
    kz = np.zeros(case.k_pool.shape, np.uint8)
    kp8, vp8 = of.kv_write_fp8_ref(kz, kz, bits(case.k_new), bits(case.v_new), case.cu_new.numpy(),
                                   case.start_pos.numpy(), case.block_tables.numpy(), 16, ks, vs)
    bt, cu, sp = case.block_tables.numpy(), case.cu_new.numpy(), case.start_pos.numpy()
    kn = bits(case.k_new)
    for b in range(3):
        for t in range(int(cu[b]), int(cu[b + 1])):
            pos = int(sp[b]) + t - int(cu[b])
            page = int(bt[b, pos // 16])
            for h in range(2):
                assert np.array_equal(kp8[page, pos % 16, h], of.quantize_ref(kn[t, h], ks[page, h]))
    # equal per-page scales reproduce the per-pool write
    k1, v1 = of.kv_write_fp8_ref(kz, kz, bits(case.k_new), bits(case.v_new), cu, sp, bt, 16,
                                 np.full((P, 2), 0.05, np.float32), np.full((P, 2), 0.02, np.float32))
    k2, v2 = of.kv_write_fp8_ref(kz, kz, bits(case.k_new), bits(case.v_new), cu, sp, bt, 16,
                                 0.05, 0.02)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def test_planted_page_scale_mistake_is_caught(monkeypatch):
    """A quantiser that takes the scale of the neighbouring page must fail the brute force."""
    real = of.page_scales
    monkeypatch.setattr(of, "page_scales",
                        lambda s, ndim=4: real(np.roll(np.asarray(s), 1, axis=0), ndim))
    with pytest.raises(AssertionError):
        test_page_scales_match_brute_force_per_element()
