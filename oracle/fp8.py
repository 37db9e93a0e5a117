"""FP8 (E4M3) key/value pages: the quantiser and its inverse, on the CPU.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

The pages name FP8 quantisation as a fusion target at KV-cache insertion
("The Stack Below the Stack (Part 2)", section 2.1, the fused inverse-RoPE plus
FP8 quantisation kernel) and FP8 KV as one ingredient of a serving recipe (the
same page, its closing "Part 3" pointer).  They fix neither the format nor the
scaling.  Readings used here (restated in the design notes):

F1  Format: the OCP 8-bit E4M3 ("fn") encoding -- 1 sign bit, 4 exponent bits
    with bias 7, 3 mantissa bits, subnormals, no infinities, the two codes
    S.1111.111 are NaN; largest finite magnitude 448 (1.75 * 2^8), smallest
    normal 2^-6, smallest subnormal 2^-9.
F2  Scaling: one float32 scale per pool (k_scale for K, v_scale for V), given
    by the caller.  A stored code c stands for decode(c) * scale.
F2' Finer scaling (an alternative to F2 the caller chooses): one float32 scale per
    (page, KV head), arrays k_scales / v_scales of shape [pages, Hkv].  A code
    in page p, head h stands for decode(c) * scales[p, h]; a new token's row is
    quantised with the scale of the page and head it is written to.
F3  Quantisation: y = float32(x) * float32(1 / scale) in float32 arithmetic,
    clamped to [-448, 448], then rounded to the nearest E4M3 value, ties to the
    even code (the IEEE default rounding).

The encoder below is written as the definition: it searches the table of every
finite E4M3 value for the nearest one, so no bit trick has to be trusted.
"""

from __future__ import annotations

import numpy as np

from .attention import bf16_bits_to_f64

__all__ = ["E4M3_MAX", "e4m3_decode", "e4m3_encode", "quantize_ref", "kv_write_fp8_ref",
           "dequantize_pool", "page_scales"]

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8) as float64 (F1)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, subnormal, normal)
    val = np.where((e == 15) & ((c & 0x7) == 7), np.nan, val)
    return sign * val


# all non-negative finite codes in increasing value order (code order is value order)
_POS_CODES = np.arange(0x7F, dtype=np.uint8)            # 0x00 .. 0x7E
_POS_VALUES = e4m3_decode(_POS_CODES)


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each finite value with |x| <= 448, ties to the even
    code (F3).  NaN maps to 0x7F; magnitudes above 448 are an error (the
    quantiser clamps before encoding)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x[~np.isnan(x)]) > E4M3_MAX):
        raise ValueError("e4m3_encode: |x| > 448 (clamp first)")
    a = np.abs(np.nan_to_num(x, nan=0.0))
    hi = np.searchsorted(_POS_VALUES, a, side="left")     # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(a == _POS_VALUES[hi], _POS_CODES[hi], code).astype(np.uint8)
    code = np.where(np.signbit(x) & (code != 0), code | 0x80, code).astype(np.uint8)
    code = np.where(np.signbit(x) & (code == 0), np.uint8(0x80), code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def page_scales(scales, ndim: int = 4) -> np.ndarray:
    """Per-(page, KV head) scales [pages, Hkv] (F2') shaped to broadcast over a pool
    [pages, page_size, Hkv, D]; a scalar (F2) is returned as a float32 scalar."""
    s = np.asarray(scales, dtype=np.float32)
    if s.ndim == 0:
        return s
    if s.ndim != 2:
        raise ValueError("per-page scales must be [pages, Hkv]")
    return s[:, None, :, None] if ndim == 4 else s


def quantize_ref(x, scale) -> np.ndarray:
    """E4M3 codes of bf16 values x (uint16 bit patterns or floats) under a pool
    scale (F2, F3), or under per-element scales broadcast against x (F2'): the
    reciprocal of each scale is taken in float32, as for a pool scale."""
    xf = bf16_bits_to_f64(x).astype(np.float32)
    inv = np.float32(1.0) / np.asarray(scale, dtype=np.float32)
    y = (xf * inv).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(y.astype(np.float64))


def dequantize_pool(codes, scale) -> np.ndarray:
    """float64 values a code pool [pages, page_size, Hkv, D] stands for:
    decode(c) * scale, with one scale per pool (F2) or per (page, KV head) (F2')."""
    return e4m3_decode(codes) * page_scales(scale).astype(np.float64)


def kv_write_fp8_ref(k_pool, v_pool, k_new, v_new, cu_new, start_pos, block_tables,
                     page_size: int, k_scale, v_scale):
    """The page write of "Inside Ion", "IonAttention in One Paragraph" (token t of
    sequence b goes to page block_tables[b][pos // page_size], slot pos % page_size)
    with the quantisation fused in ("The Stack Below the Stack (Part 2)", 2.1).
    Pools are uint8 code arrays [P, page_size, Hkv, D]; returns new arrays.  The
    scales are one float per pool (F2), or [P, Hkv] arrays (F2'): token t's heads are
    then quantised with the scales of the page it lands in."""
    kp = np.array(k_pool, dtype=np.uint8, copy=True)
    vp = np.array(v_pool, dtype=np.uint8, copy=True)
    ks, vs = np.asarray(k_scale, np.float32), np.asarray(v_scale, np.float32)
    k_new, v_new = np.asarray(k_new), np.asarray(v_new)
    cu = np.asarray(cu_new)
    for b in range(len(cu) - 1):
        for t in range(int(cu[b]), int(cu[b + 1])):
            pos = int(start_pos[b]) + (t - int(cu[b]))
            page = int(block_tables[b][pos // page_size])
            ksc = ks if ks.ndim == 0 else ks[page][:, None]        # [Hkv, 1] per head
            vsc = vs if vs.ndim == 0 else vs[page][:, None]
            kp[page, pos % page_size] = quantize_ref(k_new[t], ksc)
            vp[page, pos % page_size] = quantize_ref(v_new[t], vsc)
    return kp, vp
