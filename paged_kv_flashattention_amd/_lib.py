"""ctypes loader for libpaged_attn.so: argument types of every exported symbol.

The library is built in-tree (``python -m paged_kv_flashattention_amd.build``);
nothing here compiles or falls back.  A missing library is an error.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpaged_attn.so")

c_i32 = ctypes.c_int32
c_vp = ctypes.c_void_p
c_fp = ctypes.c_void_p          # float*, passed as raw device addresses
c_size = ctypes.c_size_t
c_float = ctypes.c_float

class DecodeOpts(ctypes.Structure):
    """pa_decode_opts"""
    _fields_ = [("num_splits", ctypes.c_int32), ("window_left", ctypes.c_int32),
                ("kv_fp8", ctypes.c_int32), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float), ("alibi_slopes", ctypes.c_void_p),
                ("kernel_start_event", ctypes.c_void_p), ("kernel_stop_event", ctypes.c_void_p),
                ("key_lo", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
                ("v_scales", ctypes.c_void_p), ("block_map", ctypes.c_void_p),
                ("block_map_k_blocks", ctypes.c_int32)]


class PrefillOpts(ctypes.Structure):
    """pa_prefill_opts"""
    _fields_ = [("causal", ctypes.c_int32), ("window_left", ctypes.c_int32),
                ("num_splits", ctypes.c_int32), ("alibi_slopes", ctypes.c_void_p),
                ("kv_fp8", ctypes.c_int32), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float), ("kernel_start_event", ctypes.c_void_p),
                ("kernel_stop_event", ctypes.c_void_p), ("key_lo", ctypes.c_void_p),
                ("key_hi", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
                ("v_scales", ctypes.c_void_p), ("persistent", ctypes.c_int32),
                ("block_map", ctypes.c_void_p), ("block_map_q_blocks", ctypes.c_int32),
                ("block_map_k_blocks", ctypes.c_int32)]


class MixedPrefill(ctypes.Structure):
    """pa_mixed_prefill"""
    _fields_ = [("out", ctypes.c_void_p), ("lse_out", ctypes.c_void_p), ("q", ctypes.c_void_p),
                ("cu_seqlens_q", ctypes.c_void_p), ("seq_lens_k", ctypes.c_void_p),
                ("block_tables", ctypes.c_void_p), ("B", ctypes.c_int32), ("Tq", ctypes.c_int32),
                ("max_q_len", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("num_splits", ctypes.c_int32)]


class MixedDecode(ctypes.Structure):
    """pa_mixed_decode"""
    _fields_ = [("out", ctypes.c_void_p), ("lse_out", ctypes.c_void_p), ("q", ctypes.c_void_p),
                ("block_tables", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("B", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("num_splits", ctypes.c_int32)]


class MixedFp8(ctypes.Structure):
    """pa_mixed_fp8"""
    _fields_ = [("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p)]


c_dopts = ctypes.POINTER(DecodeOpts)
c_popts = ctypes.POINTER(PrefillOpts)
c_mpf = ctypes.POINTER(MixedPrefill)
c_mdec = ctypes.POINTER(MixedDecode)
c_mfp8 = ctypes.POINTER(MixedFp8)

# name -> (restype, argtypes); mirrors include/paged_attn.h
SIGNATURES = {
    "kv_page_write": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                              c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp]),
    "kv_page_write_fp8": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                  c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                  c_float, c_float, c_vp]),
    "kv_page_write_fp8_scales": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                         c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                         c_fp, c_fp, c_vp]),
    "paged_attn_decode_num_splits": (c_i32, [c_i32, c_i32, c_i32]),
    "paged_attn_decode_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "paged_attn_decode": (c_i32, [c_vp, c_fp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                  c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                  c_float, c_i32, c_i32, c_vp, c_size, c_vp]),
    "paged_attn_decode_noalloc": (c_i32, [c_vp, c_fp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                          c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                          c_float, c_i32, c_i32, c_vp]),
    "paged_attn_decode_fp8": (c_i32, [c_vp, c_fp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                      c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                      c_float, c_float, c_float, c_i32, c_i32, c_vp, c_size,
                                      c_vp]),
    "paged_attn_decode_partials": (c_i32, [c_fp, c_fp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                           c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                           c_float, c_i32, c_i32, c_vp]),
    "paged_attn_splitk_reduce": (c_i32, [c_vp, c_fp, c_fp, c_fp, c_i32, c_i32, c_i32, c_vp]),
    "paged_attn_prefill_varlen": (c_i32, [c_vp, c_fp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                          c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                          c_i32, c_i32, c_float, c_i32, c_vp]),
    "paged_attn_prefill_varlen_splitk": (c_i32, [c_vp, c_fp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                                 c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                                 c_i32, c_i32, c_i32, c_float, c_i32, c_i32,
                                                 c_vp, c_size, c_vp]),
    "paged_attn_prefill_num_splits": (c_i32, [c_i32, c_i32, c_i32]),
    "paged_attn_prefill_plan_splits": (c_i32, [c_i32, c_vp, c_vp, c_i32, c_i32, c_i32]),
    "paged_attn_prefill_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "paged_attn_decode_ex": (c_i32, [c_vp, c_fp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                     c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                     c_float, c_i32, c_dopts, c_vp, c_size, c_vp]),
    "paged_attn_decode_ex_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32, c_i32,
                                                      c_dopts]),
    "paged_attn_prefill_ex": (c_i32, [c_vp, c_fp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                      c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                      c_i32, c_float, c_popts, c_vp, c_size, c_vp]),
    "paged_attn_prefill_ex_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32, c_i32,
                                                       c_popts]),
    "paged_attn_mixed_workspace_bytes": (c_size, [c_mpf, c_mdec, c_mfp8, c_i32, c_i32, c_i32]),
    "paged_attn_mixed": (c_i32, [c_mpf, c_mdec, c_mfp8, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                 c_i32, c_float, c_vp, c_size, c_vp]),
    "pa_status_string": (ctypes.c_char_p, [c_i32]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_describe_launch": (ctypes.c_char_p, []),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m paged_kv_flashattention_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
