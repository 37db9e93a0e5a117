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
