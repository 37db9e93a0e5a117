"""Exact attention over a paged KV cache on AMD MI355X (gfx950).

A thin binding over the C ABI of ``libpaged_attn.so`` (``include/paged_attn.h``):
argument checks and marshalling only.  Every step of the computation runs in the
library's HIP kernels; torch supplies device memory and the current stream.

Entry points (same names as the C ABI):

* :func:`kv_page_write`      -- place new tokens' K/V into their pages;
* :func:`kv_page_write_fp8`  -- the same, quantising into FP8 E4M3 pools;
* :func:`paged_attn_decode`  -- one query row per sequence, split-K + merge;
* :func:`paged_attn_decode_fp8` -- decode over FP8 E4M3 pools;
* :func:`paged_attn_decode_partials` -- decode's per-partition results only;
* :func:`paged_attn_splitk_reduce` -- the merge on its own;
* :func:`paged_attn_prefill_varlen` -- ragged (causal) prefill on MFMA;
* :func:`paged_attn_prefill_varlen_splitk` -- the same with long key ranges cut
  into parts computed by separate work-groups and merged;
* :func:`paged_attn_prefill_varlen_fp8` -- prefill over FP8 E4M3 pools.

Data contract: bf16 Q / K / V / outputs, int32 indices (int64 is refused, not
cast), fp32 lse, contiguous tensors on one GPU.  FP8 pools are uint8 (or
torch.float8_e4m3fn) tensors of E4M3 codes with one float32 scale per pool (floats)
or one per (page, KV head) (float32 tensors [num_pages, Hkv] on the pools' GPU).
An unsupported configuration raises; there is no fallback path.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib

__all__ = [
    "PagedAttnError", "kv_page_write", "kv_page_write_fp8", "paged_attn_decode",
    "paged_attn_decode_fp8", "paged_attn_decode_partials",
    "paged_attn_splitk_reduce",
    "paged_attn_prefill_varlen", "paged_attn_prefill_varlen_splitk",
    "paged_attn_prefill_varlen_fp8", "prefill_num_splits",
    "prefill_workspace_bytes", "decode_num_splits", "decode_workspace_bytes",
    "describe_launch", "library_path", "load_library", "paged_attn_mixed",
    "mixed_workspace_bytes",
]

PA_STATUS = {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_UNSUPPORTED",
             4: "PA_ERR_MISALIGNED", 5: "PA_ERR_WORKSPACE", 6: "PA_ERR_LAUNCH"}


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{PA_STATUS.get(status, status)}: {detail}")


_RECORDER = None


def load_library():
    return _RECORDER if _RECORDER is not None else _lib.load()


class _Recorder:
    """Stands in for the library while prepared() runs a call: forwards every C call
    and keeps the launching ones with their marshalled arguments."""

    _HOST_ONLY = ("_bytes", "_num_splits", "_plan_splits")

    def __init__(self, lib):
        self._lib = lib
        self.launches = []
        self.keep = []          # buffers the binding allocated during the recorded call

    def __getattr__(self, name):
        fn = getattr(self._lib, name)
        if name.startswith("pa_") or name.endswith(self._HOST_ONLY):
            return fn

        def call(*args):
            self.launches.append((fn, args))
            return fn(*args)
        return call


def prepared(call):
    """Run ``call`` -- a function that makes calls of this module -- once, and return a
    function that repeats exactly its C calls with the same marshalled arguments
    (pointers, sizes, the stream current at preparation) without the Python-side
    checks, for launch loops whose host cost matters.  The tensors ``call`` passed in
    must stay alive, and keep their storage, while the returned function is used;
    buffers the binding allocated itself during ``call`` (outputs, workspaces) are
    held by the returned function, so their memory is never handed out again while
    it may still run."""
    global _RECORDER
    rec = _Recorder(_lib.load())
    _RECORDER = rec
    try:
        call()
    finally:
        _RECORDER = None
    launches = list(rec.launches)
    keep = list(rec.keep)

    def run():
        _ = keep
        for fn, args in launches:
            status = fn(*args)
            if status != 0:
                _check(status)
    return run


def library_path() -> str:
    return _lib.LIB_PATH


def describe_launch() -> str:
    return load_library().pa_describe_launch().decode()


def _check(status: int):
    if status != 0:
        raise PagedAttnError(status, load_library().pa_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _internal(t: torch.Tensor, stream) -> torch.Tensor:
    """Book-keeping for a buffer the binding allocated for one call (an output or a
    workspace the caller did not pass).  torch's caching allocator ties a block to
    the stream current at allocation; when the launch stream is another one, the
    block is marked in use there too, so that it is not handed to the current
    stream's next allocation while the launch stream's kernels still read or write
    it.  While prepared() records a call, the buffer is also kept alive by the
    recording, whose replays write into it."""
    if _RECORDER is not None:
        _RECORDER.keep.append(t)
    if stream is not None:
        handle = _stream(stream)
        if handle != torch.cuda.current_stream(t.device).cuda_stream:
            s = stream if isinstance(stream, torch.cuda.Stream) else \
                torch.cuda.ExternalStream(handle, device=t.device)
            t.record_stream(s)
    return t


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int, device):
    _need_dtype(t, name, dtype)
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _need_dtype(t: torch.Tensor, name: str, dtype: torch.dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype} (no implicit casts)")


FP8_POOL_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def _need_fp8_dtype(t, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in FP8_POOL_DTYPES:
        raise TypeError(f"{name} must hold E4M3 codes as uint8 or float8_e4m3fn, got {t.dtype}")


def _need_fp8_pool(t, name: str, device):
    _need_fp8_dtype(t, name)
    if t.dim() != 4:
        raise ValueError(f"{name} must have 4 dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


class _PageScales:
    """FP8 scales per (page, KV head): device float32 tensors [num_pages, Hkv]."""

    def __init__(self, k, v):
        self.k, self.v = k, v

    def check(self, pool_shape, dev):
        P, _, Hkv, _ = pool_shape
        for t, name in ((self.k, "k_scale"), (self.v, "v_scale")):
            _need(t, name, torch.float32, 2, dev)
            if tuple(t.shape) != (P, Hkv):
                raise ValueError(f"{name} per page must be [num_pages={P}, Hkv={Hkv}], got "
                                 f"{tuple(t.shape)}")
        return self.k.data_ptr(), self.v.data_ptr()


def _scales(k_scale, v_scale):
    """One float32 scale per pool (floats), or per (page, KV head) (two tensors)."""
    if isinstance(k_scale, torch.Tensor) or isinstance(v_scale, torch.Tensor):
        if not (isinstance(k_scale, torch.Tensor) and isinstance(v_scale, torch.Tensor)):
            raise TypeError("k_scale and v_scale must both be floats or both be tensors")
        _dtypes((k_scale, "k_scale", torch.float32), (v_scale, "v_scale", torch.float32))
        return _PageScales(k_scale, v_scale)
    ks, vs = float(k_scale), float(v_scale)
    if not (0.0 < ks < float("inf") and 0.0 < vs < float("inf")):
        raise ValueError(f"k_scale and v_scale must be positive and finite, got {ks}, {vs}")
    return ks, vs


def _pool_scales(scales):
    """(k_scale, v_scale) floats of the C call: 1 with scales per page (ignored)."""
    return (1.0, 1.0) if isinstance(scales, _PageScales) else scales


def _dtypes(*specs):
    """Check every argument's dtype before anything else, so a dtype mistake is
    reported as such whatever else is wrong."""
    for t, name, dtype in specs:
        if t is not None:
            _need_dtype(t, name, dtype)


def _validate_tables(block_tables, seq_lens, num_pages, page_size, what="seq_lens"):
    bt = block_tables.cpu()
    lens = seq_lens.cpu()
    max_pages = bt.shape[1]
    for b in range(bt.shape[0]):
        L = int(lens[b])
        if L < 0 or L > max_pages * page_size:
            raise ValueError(f"{what}[{b}]={L} does not fit a table row of {max_pages} pages")
        n = -(-L // page_size)
        if n and (int(bt[b, :n].min()) < 0 or int(bt[b, :n].max()) >= num_pages):
            raise ValueError(f"block_tables row {b} references a page outside [0, {num_pages})")


def kv_page_write(k_pool, v_pool, k_new, v_new, cu_new, start_pos, block_tables,
                  stream=None, validate: bool = False) -> None:
    """Write k_new/v_new [T, Hkv, D] into the pools in place (see kv_page_write in C)."""
    _kv_write(None, k_pool, v_pool, k_new, v_new, cu_new, start_pos, block_tables, stream,
              validate)


def kv_page_write_fp8(k_pool, v_pool, k_new, v_new, cu_new, start_pos, block_tables,
                      k_scale, v_scale, stream=None, validate: bool = False) -> None:
    """Quantise k_new/v_new [T, Hkv, D] bf16 to E4M3 codes and write them into the
    uint8 pools in place: under one scale per pool (floats; kv_page_write_fp8 in C)
    or one per (page, KV head) (float32 tensors [num_pages, Hkv] on the device;
    kv_page_write_fp8_scales in C)."""
    _kv_write(_scales(k_scale, v_scale), k_pool, v_pool, k_new, v_new, cu_new, start_pos,
              block_tables, stream, validate)


def _kv_write(scales, k_pool, v_pool, k_new, v_new, cu_new, start_pos, block_tables, stream,
              validate):
    if scales is None:
        _dtypes((k_pool, "k_pool", torch.bfloat16), (v_pool, "v_pool", torch.bfloat16))
    else:
        _need_fp8_dtype(k_pool, "k_pool")
        _need_fp8_dtype(v_pool, "v_pool")
    _dtypes((k_new, "k_new", torch.bfloat16), (v_new, "v_new", torch.bfloat16),
            (cu_new, "cu_new", torch.int32), (start_pos, "start_pos", torch.int32),
            (block_tables, "block_tables", torch.int32))
    dev = k_pool.device
    if scales is None:
        _need(k_pool, "k_pool", torch.bfloat16, 4, None)
        _need(v_pool, "v_pool", torch.bfloat16, 4, dev)
    else:
        _need_fp8_pool(k_pool, "k_pool", None)
        _need_fp8_pool(v_pool, "v_pool", dev)
    _need(k_new, "k_new", torch.bfloat16, 3, dev)
    _need(v_new, "v_new", torch.bfloat16, 3, dev)
    _need(cu_new, "cu_new", torch.int32, 1, dev)
    _need(start_pos, "start_pos", torch.int32, 1, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    P, ps, Hkv, D = k_pool.shape
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool shapes differ")
    T = k_new.shape[0]
    if k_new.shape != (T, Hkv, D) or v_new.shape != (T, Hkv, D):
        raise ValueError(f"k_new/v_new must be [T, {Hkv}, {D}]")
    B = start_pos.shape[0]
    if cu_new.shape[0] != B + 1 or block_tables.shape[0] != B:
        raise ValueError("cu_new must be [B+1] and block_tables [B, max_pages]")
    if validate:
        cu = cu_new.cpu()
        sp = start_pos.cpu()
        if int(cu[0]) != 0 or int(cu[-1]) != T or bool((cu[1:] < cu[:-1]).any()):
            raise ValueError("cu_new must be non-decreasing from 0 to T")
        ends = sp + (cu[1:] - cu[:-1])
        _validate_tables(block_tables, ends, P, ps, "start_pos + new tokens")
        seen = set()
        bt = block_tables.cpu()
        for b in range(B):
            for pos in range(int(sp[b]), int(ends[b])):
                key = (int(bt[b, pos // ps]), pos % ps)
                if key in seen:
                    raise ValueError(f"two new tokens write page {key[0]} slot {key[1]}")
                seen.add(key)
    args = (_ptr(k_pool), _ptr(v_pool), _ptr(k_new), _ptr(v_new), _ptr(cu_new),
            _ptr(start_pos), _ptr(block_tables), B, T, block_tables.shape[1], P, ps, Hkv, D)
    lib = load_library()
    with torch.cuda.device(dev):
        if scales is None:
            _check(lib.kv_page_write(*args, _stream(stream)))
        elif isinstance(scales, _PageScales):
            kp_, vp_ = scales.check(k_pool.shape, dev)
            _check(lib.kv_page_write_fp8_scales(*args, kp_, vp_, _stream(stream)))
        else:
            _check(lib.kv_page_write_fp8(*args, scales[0], scales[1], _stream(stream)))


def decode_num_splits(B: int, Hkv: int, max_seq_len: int) -> int:
    return int(load_library().paged_attn_decode_num_splits(B, Hkv, max_seq_len))


def decode_workspace_bytes(B, Hq, Hkv, D, max_seq_len, num_splits=0) -> int:
    """Workspace bytes for paged_attn_decode (scratch; no initialisation needed)."""
    return int(load_library().paged_attn_decode_workspace_bytes(B, Hq, Hkv, D, max_seq_len,
                                                                num_splits))


def paged_attn_decode(q, k_pool, v_pool, block_tables, seq_lens, softmax_scale: float,
                      max_seq_len: Optional[int] = None, num_splits: int = 0,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, return_lse: bool = False,
                      stream=None, validate: bool = False, window_left: int = 0,
                      alibi_slopes: Optional[torch.Tensor] = None, kernel_events=None,
                      key_lo: Optional[torch.Tensor] = None,
                      block_map: Optional[torch.Tensor] = None):
    """Decode attention: q [B, Hq, D] against each sequence's paged history.

    ``max_seq_len`` is a host-side bound of ``seq_lens``; if omitted it is read
    from the device (a synchronisation).  Returns out [B, Hq, D] bf16, and the
    natural-log lse [B, Hq] fp32 as well when ``return_lse``.  ``window_left`` = w > 0
    restricts each row to its last w keys (sliding window; see paged_attn_decode_ex);
    ``alibi_slopes`` (float32 [Hq] on the device) adds slope_h * (j - p) to the scores.
    ``kernel_events`` = (start, stop) torch.cuda.Event pair (timing enabled, recorded
    once already) that the partition kernel's dispatch stamps with its own start and
    end (see pa_decode_opts).  ``key_lo`` (int32 [B] on the device): document masks,
    the first key of the document each decode row belongs to.  ``block_map`` (uint8
    [B, key blocks] on the device): the row of sequence b sees key j only if
    block_map[b, j // 64] is nonzero (a mask in block form; blocks outside the map
    count as zero).
    """
    return _decode(None, q, k_pool, v_pool, block_tables, seq_lens, softmax_scale, max_seq_len,
                   num_splits, out, lse, workspace, return_lse, stream, validate, window_left,
                   alibi_slopes, kernel_events, key_lo, block_map)


def paged_attn_decode_fp8(q, k_pool, v_pool, block_tables, seq_lens, softmax_scale: float,
                          k_scale, v_scale, max_seq_len: Optional[int] = None,
                          num_splits: int = 0, out: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, return_lse: bool = False,
                          stream=None, validate: bool = False, window_left: int = 0,
                          alibi_slopes: Optional[torch.Tensor] = None, kernel_events=None,
                          key_lo: Optional[torch.Tensor] = None,
                          block_map: Optional[torch.Tensor] = None):
    """Decode attention over FP8 E4M3 pools (uint8 codes): keys stand for
    decode(code) * k_scale, values for decode(code) * v_scale, with one scale per pool
    (floats) or per (page, KV head) (float32 tensors [num_pages, Hkv] on the device).
    Arguments and results are paged_attn_decode's."""
    return _decode(_scales(k_scale, v_scale), q, k_pool, v_pool, block_tables, seq_lens,
                   softmax_scale, max_seq_len, num_splits, out, lse, workspace, return_lse,
                   stream, validate, window_left, alibi_slopes, kernel_events, key_lo,
                   block_map)


def _window(window_left) -> int:
    w = int(window_left)
    if w < 0:
        raise ValueError(f"window_left must be >= 0, got {w}")
    return w


def _alibi(slopes, Hq, dev):
    """Device pointer of an ALiBi slope vector (float32 [Hq]), or None."""
    if slopes is None:
        return None
    _need_dtype(slopes, "alibi_slopes", torch.float32)
    _need(slopes, "alibi_slopes", torch.float32, 1, dev)
    if slopes.shape[0] != Hq:
        raise ValueError(f"alibi_slopes must have Hq={Hq} entries, got {slopes.shape[0]}")
    return slopes.data_ptr()


def _events(kernel_events):
    """(start, stop) raw hipEvent_t handles from a pair of torch.cuda.Event (created,
    i.e. recorded at least once, with enable_timing=True) or of ints; (None, None)."""
    if kernel_events is None:
        return None, None
    if len(kernel_events) != 2:
        raise ValueError("kernel_events must be a (start, stop) pair")
    out = []
    for ev in kernel_events:
        h = int(ev) if isinstance(ev, int) else int(ev.cuda_event)
        if h == 0:
            raise ValueError("kernel_events: a HIP event is created when first recorded; "
                             "record each event once before passing it")
        out.append(h)
    return tuple(out)


def _decode(scales, q, k_pool, v_pool, block_tables, seq_lens, softmax_scale, max_seq_len,
            num_splits, out, lse, workspace, return_lse, stream, validate, window_left=0,
            alibi_slopes=None, kernel_events=None, key_lo=None, block_map=None):
    window_left = _window(window_left)
    if scales is None:
        _dtypes((k_pool, "k_pool", torch.bfloat16), (v_pool, "v_pool", torch.bfloat16))
    else:
        _need_fp8_dtype(k_pool, "k_pool")
        _need_fp8_dtype(v_pool, "v_pool")
    _dtypes((q, "q", torch.bfloat16), (block_tables, "block_tables", torch.int32),
            (seq_lens, "seq_lens", torch.int32), (out, "out", torch.bfloat16),
            (lse, "lse", torch.float32))
    dev = q.device
    _need(q, "q", torch.bfloat16, 3, None)
    if scales is None:
        _need(k_pool, "k_pool", torch.bfloat16, 4, dev)
        _need(v_pool, "v_pool", torch.bfloat16, 4, dev)
    else:
        _need_fp8_pool(k_pool, "k_pool", dev)
        _need_fp8_pool(v_pool, "v_pool", dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    B, Hq, D = q.shape
    P, ps, Hkv, Dk = k_pool.shape
    if Dk != D or v_pool.shape != k_pool.shape:
        raise ValueError("pool shapes do not match q")
    if seq_lens.shape[0] != B or block_tables.shape[0] != B:
        raise ValueError("seq_lens must be [B] and block_tables [B, max_pages]")
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B else 0
    if validate:
        _validate_tables(block_tables, seq_lens, P, ps)
        if B and int(seq_lens.max().item()) > max_seq_len:
            raise ValueError("max_seq_len is below a sequence length")
    if out is None:
        out = _internal(torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev), stream)
    else:
        _need(out, "out", torch.bfloat16, 3, dev)
    if return_lse and lse is None:
        lse = _internal(torch.empty((B, Hq), dtype=torch.float32, device=dev), stream)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
    lib = load_library()
    alibi_ptr = _alibi(alibi_slopes, Hq, dev)
    lo_ptr = None
    if key_lo is not None:
        _need(key_lo, "key_lo", torch.int32, 1, dev)
        if key_lo.shape[0] != B:
            raise ValueError(f"key_lo must have B={B} entries")
        if validate:
            lo_h, lens_h = key_lo.cpu(), seq_lens.cpu()
            if bool((lo_h < 0).any()) or bool((lo_h > lens_h).any()):
                raise ValueError("key_lo must lie in [0, seq_lens]")
        lo_ptr = key_lo.data_ptr()
    bm_ptr, bm_k = None, 0
    if block_map is not None:
        _need(block_map, "block_map", torch.uint8, 2, dev)
        if block_map.shape[0] != B:
            raise ValueError(f"block_map must be [B={B}, key blocks]")
        bm_ptr, bm_k = block_map.data_ptr(), block_map.shape[1]
    ev0, ev1 = _events(kernel_events)
    ksp = vsp = None
    if isinstance(scales, _PageScales):
        ksp, vsp = scales.check(k_pool.shape, dev)
    opts = _lib.DecodeOpts(int(num_splits), window_left, 0 if scales is None else 1,
                           *(_pool_scales(scales) if scales is not None else (1.0, 1.0)),
                           alibi_ptr, ev0, ev1, lo_ptr, ksp, vsp, bm_ptr, bm_k)
    need = int(lib.paged_attn_decode_ex_workspace_bytes(B, Hq, Hkv, D, int(max_seq_len),
                                                        ctypes.byref(opts)))
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1, dev)
    elif need:
        workspace = _internal(torch.empty(need, dtype=torch.uint8, device=dev), stream)
    ws_bytes = 0 if workspace is None else workspace.numel()
    head = (_ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
            _ptr(seq_lens), B, block_tables.shape[1], P, ps, Hq, Hkv, D, float(softmax_scale))
    tail = (int(max_seq_len), int(num_splits), _ptr(workspace), ws_bytes, _stream(stream))
    with torch.cuda.device(dev):
        if (window_left or alibi_ptr is not None or ev0 is not None or lo_ptr is not None
                or ksp is not None or bm_ptr is not None):
            _check(lib.paged_attn_decode_ex(*head, int(max_seq_len), ctypes.byref(opts),
                                            *tail[2:]))
        elif scales is None:
            _check(lib.paged_attn_decode(*head, *tail))
        else:
            _check(lib.paged_attn_decode_fp8(*head, scales[0], scales[1], *tail))
    return (out, lse) if return_lse else out


def paged_attn_decode_partials(q, k_pool, v_pool, block_tables, seq_lens, softmax_scale: float,
                               num_splits: int, max_seq_len: Optional[int] = None,
                               partial_out: Optional[torch.Tensor] = None,
                               partial_lse: Optional[torch.Tensor] = None, stream=None):
    """Per-partition decode results: partial_out [B*Hq, S, D] fp32, partial_lse [B*Hq, S]."""
    _dtypes((q, "q", torch.bfloat16), (k_pool, "k_pool", torch.bfloat16),
            (v_pool, "v_pool", torch.bfloat16), (block_tables, "block_tables", torch.int32),
            (seq_lens, "seq_lens", torch.int32), (partial_out, "partial_out", torch.float32),
            (partial_lse, "partial_lse", torch.float32))
    dev = q.device
    _need(q, "q", torch.bfloat16, 3, None)
    _need(k_pool, "k_pool", torch.bfloat16, 4, dev)
    _need(v_pool, "v_pool", torch.bfloat16, 4, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    B, Hq, D = q.shape
    P, ps, Hkv, Dk = k_pool.shape
    if Dk != D or v_pool.shape != k_pool.shape:
        raise ValueError("pool shapes do not match q")
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B else 0
    S = int(num_splits)
    if partial_out is None:
        partial_out = _internal(torch.empty((B * Hq, S, D), dtype=torch.float32, device=dev),
                                stream)
    _need(partial_out, "partial_out", torch.float32, 3, dev)
    if partial_lse is None:
        partial_lse = _internal(torch.empty((B * Hq, S), dtype=torch.float32, device=dev),
                                stream)
    _need(partial_lse, "partial_lse", torch.float32, 2, dev)
    if tuple(partial_out.shape) != (B * Hq, S, D) or tuple(partial_lse.shape) != (B * Hq, S):
        raise ValueError("partials must be [B*Hq, S, D] and [B*Hq, S]")
    with torch.cuda.device(dev):
        _check(load_library().paged_attn_decode_partials(
            _ptr(partial_out), _ptr(partial_lse), _ptr(q), _ptr(k_pool), _ptr(v_pool),
            _ptr(block_tables), _ptr(seq_lens), B, block_tables.shape[1], P, ps, Hq, Hkv, D,
            float(softmax_scale), int(max_seq_len), S, _stream(stream)))
    return partial_out, partial_lse


def paged_attn_splitk_reduce(partial_out, partial_lse, out=None, lse=None, stream=None,
                             want_lse: bool = True):
    """Merge partial_out [R, S, D] fp32 with partial_lse [R, S] fp32 -> (out bf16, lse fp32).
    With want_lse=False and no ``lse`` given, no lse is written (returned as None)."""
    _dtypes((partial_out, "partial_out", torch.float32), (partial_lse, "partial_lse", torch.float32),
            (out, "out", torch.bfloat16), (lse, "lse", torch.float32))
    dev = partial_out.device
    _need(partial_out, "partial_out", torch.float32, 3, None)
    _need(partial_lse, "partial_lse", torch.float32, 2, dev)
    R, S, D = partial_out.shape
    if partial_lse.shape != (R, S):
        raise ValueError("partial_lse must be [R, S]")
    if out is None:
        out = _internal(torch.empty((R, D), dtype=torch.bfloat16, device=dev), stream)
    _need(out, "out", torch.bfloat16, 2, dev)
    if lse is None and want_lse:
        lse = _internal(torch.empty((R,), dtype=torch.float32, device=dev), stream)
    if lse is not None:
        _need(lse, "lse", torch.float32, 1, dev)
    with torch.cuda.device(dev):
        _check(load_library().paged_attn_splitk_reduce(
            _ptr(out), _ptr(lse), _ptr(partial_out), _ptr(partial_lse), R, S, D,
            _stream(stream)))
    return out, lse


def paged_attn_prefill_varlen(q, k_pool, v_pool, cu_seqlens_q, seq_lens_k, block_tables,
                              softmax_scale: float, causal: bool = True,
                              max_q_len: Optional[int] = None,
                              out: Optional[torch.Tensor] = None,
                              lse: Optional[torch.Tensor] = None, return_lse: bool = False,
                              stream=None, validate: bool = False, window_left: int = 0,
                              alibi_slopes: Optional[torch.Tensor] = None, kernel_events=None,
                              key_ranges=None, persistent: bool = False,
                              block_map: Optional[torch.Tensor] = None):
    """Ragged prefill: q [Tq, Hq, D] rows of B sequences over their paged keys.

    ``max_q_len`` is a host-side bound of the per-sequence query counts; if
    omitted it is read from the device (a synchronisation).  ``window_left`` = w > 0
    restricts the row at position p to keys j > p - w (sliding window);
    ``alibi_slopes`` (float32 [Hq] on the device) adds slope_h * (j - p) to the scores.
    ``kernel_events`` as paged_attn_decode's, for the prefill kernel.
    ``key_ranges`` = (key_lo, key_hi), int32 [Tq] each on the device: document masks,
    row t sees keys key_lo[t] <= j < key_hi[t] of its sequence only.
    ``persistent``: persistent work-groups with next-item prefetch (the ``persistent``
    field of pa_prefill_opts; plain bf16 variant with 256-row tiles, else ignored).
    ``block_map``: uint8 [B, query blocks, key blocks] on the device, a mask in block
    form -- row i of sequence b's query run sees key j only if
    block_map[b, i // 64, j // 64] is nonzero (entries outside the map count as zero),
    on top of the other masks.
    """
    return _prefill(None, q, k_pool, v_pool, cu_seqlens_q, seq_lens_k, block_tables,
                    softmax_scale, causal, max_q_len, out, lse, return_lse, stream, validate,
                    window_left, alibi_slopes, kernel_events=kernel_events,
                    key_ranges=key_ranges, persistent=persistent, block_map=block_map)


def paged_attn_prefill_varlen_fp8(q, k_pool, v_pool, cu_seqlens_q, seq_lens_k, block_tables,
                                  softmax_scale: float, k_scale, v_scale,
                                  causal: bool = True, max_q_len: Optional[int] = None,
                                  num_splits: int = 1, out: Optional[torch.Tensor] = None,
                                  lse: Optional[torch.Tensor] = None,
                                  workspace: Optional[torch.Tensor] = None,
                                  return_lse: bool = False, stream=None,
                                  validate: bool = False, window_left: int = 0,
                                  alibi_slopes: Optional[torch.Tensor] = None,
                                  kernel_events=None, key_ranges=None,
                                  block_map: Optional[torch.Tensor] = None):
    """Ragged prefill over FP8 E4M3 pools (uint8 codes; keys stand for decode(code) *
    k_scale, values for decode(code) * v_scale; scales per pool as floats or per (page,
    KV head) as float32 tensors [num_pages, Hkv]), through paged_attn_prefill_ex.
    ``num_splits`` as paged_attn_prefill_varlen_splitk's (1: one pass); ``block_map``
    as paged_attn_prefill_varlen's (one pass only)."""
    return _prefill((int(num_splits), workspace), q, k_pool, v_pool, cu_seqlens_q, seq_lens_k,
                    block_tables, softmax_scale, causal, max_q_len, out, lse, return_lse, stream,
                    validate, window_left, alibi_slopes, _scales(k_scale, v_scale),
                    kernel_events, key_ranges, block_map=block_map)


def prefill_num_splits(B: int, Hq: int, max_q_len: int) -> int:
    return int(load_library().paged_attn_prefill_num_splits(B, Hq, max_q_len))


def prefill_plan_splits(q_lens, k_lens, Hq: int, causal: bool = True,
                        window_left: int = 0) -> int:
    """Key parts for paged_attn_prefill_varlen_splitk planned from host lengths
    (sequences of ints: query rows and keys per sequence); see
    paged_attn_prefill_plan_splits in C."""
    q = (ctypes.c_int32 * len(q_lens))(*[int(x) for x in q_lens])
    k = (ctypes.c_int32 * len(k_lens))(*[int(x) for x in k_lens])
    if len(q) != len(k):
        raise ValueError("q_lens and k_lens must have one entry per sequence")
    lib = load_library()
    s = int(lib.paged_attn_prefill_plan_splits(len(q), ctypes.cast(q, ctypes.c_void_p),
                                               ctypes.cast(k, ctypes.c_void_p), int(Hq),
                                               1 if causal else 0, _window(window_left)))
    if s <= 0:
        raise PagedAttnError(2, lib.pa_last_error().decode())
    return s


def prefill_workspace_bytes(B, Tq, max_q_len, Hq, D, num_splits=0) -> int:
    """Workspace bytes for paged_attn_prefill_varlen_splitk (scratch)."""
    return int(load_library().paged_attn_prefill_workspace_bytes(B, Tq, max_q_len, Hq, D,
                                                                 num_splits))


def paged_attn_prefill_varlen_splitk(q, k_pool, v_pool, cu_seqlens_q, seq_lens_k, block_tables,
                                     softmax_scale: float, causal: bool = True,
                                     max_q_len: Optional[int] = None, num_splits: int = 0,
                                     out: Optional[torch.Tensor] = None,
                                     lse: Optional[torch.Tensor] = None,
                                     workspace: Optional[torch.Tensor] = None,
                                     return_lse: bool = False, stream=None,
                                     validate: bool = False, window_left: int = 0,
                                     alibi_slopes: Optional[torch.Tensor] = None,
                                     kernel_events=None, key_ranges=None,
                                     persistent: bool = False):
    """Ragged prefill with long key ranges cut into at most ``num_splits`` parts
    (<= 0: the library's choice) and merged; see paged_attn_prefill_varlen_splitk in C.
    ``persistent`` as paged_attn_prefill_varlen's."""
    return _prefill((int(num_splits), workspace), q, k_pool, v_pool, cu_seqlens_q, seq_lens_k,
                    block_tables, softmax_scale, causal, max_q_len, out, lse, return_lse, stream,
                    validate, window_left, alibi_slopes, None, kernel_events, key_ranges,
                    persistent)


def _prefill(split, q, k_pool, v_pool, cu_seqlens_q, seq_lens_k, block_tables, softmax_scale,
             causal, max_q_len, out, lse, return_lse, stream, validate, window_left=0,
             alibi_slopes=None, scales=None, kernel_events=None, key_ranges=None,
             persistent=False, block_map=None):
    window_left = _window(window_left)
    if scales is None:
        _dtypes((k_pool, "k_pool", torch.bfloat16), (v_pool, "v_pool", torch.bfloat16))
    else:
        _need_fp8_dtype(k_pool, "k_pool")
        _need_fp8_dtype(v_pool, "v_pool")
    _dtypes((q, "q", torch.bfloat16), (cu_seqlens_q, "cu_seqlens_q", torch.int32),
            (seq_lens_k, "seq_lens_k", torch.int32), (block_tables, "block_tables", torch.int32),
            (out, "out", torch.bfloat16), (lse, "lse", torch.float32))
    dev = q.device
    _need(q, "q", torch.bfloat16, 3, None)
    if scales is None:
        _need(k_pool, "k_pool", torch.bfloat16, 4, dev)
        _need(v_pool, "v_pool", torch.bfloat16, 4, dev)
    else:
        _need_fp8_pool(k_pool, "k_pool", dev)
        _need_fp8_pool(v_pool, "v_pool", dev)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, dev)
    _need(seq_lens_k, "seq_lens_k", torch.int32, 1, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    Tq, Hq, D = q.shape
    P, ps, Hkv, Dk = k_pool.shape
    B = seq_lens_k.shape[0]
    if Dk != D or v_pool.shape != k_pool.shape:
        raise ValueError("pool shapes do not match q")
    if cu_seqlens_q.shape[0] != B + 1 or block_tables.shape[0] != B:
        raise ValueError("cu_seqlens_q must be [B+1] and block_tables [B, max_pages]")
    if max_q_len is None:
        max_q_len = int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item()) if B else 0
    if validate:
        cu = cu_seqlens_q.cpu()
        if int(cu[0]) != 0 or int(cu[-1]) != Tq or bool((cu[1:] < cu[:-1]).any()):
            raise ValueError("cu_seqlens_q must be non-decreasing from 0 to Tq")
        if B and int((cu[1:] - cu[:-1]).max()) > max_q_len:
            raise ValueError("max_q_len is below a sequence's query count")
        _validate_tables(block_tables, seq_lens_k, P, ps)
    if out is None:
        out = _internal(torch.empty((Tq, Hq, D), dtype=torch.bfloat16, device=dev), stream)
    else:
        _need(out, "out", torch.bfloat16, 3, dev)
    if return_lse and lse is None:
        lse = _internal(torch.empty((Tq, Hq), dtype=torch.float32, device=dev), stream)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
    lib = load_library()
    args = (_ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(cu_seqlens_q),
            _ptr(seq_lens_k), _ptr(block_tables), B, Tq, int(max_q_len), block_tables.shape[1],
            P, ps, Hq, Hkv, D, float(softmax_scale), 1 if causal else 0)
    alibi_ptr = _alibi(alibi_slopes, Hq, dev)
    lo_ptr = hi_ptr = None
    if key_ranges is not None:
        if len(key_ranges) != 2:
            raise ValueError("key_ranges must be a (key_lo, key_hi) pair")
        key_lo, key_hi = key_ranges
        _need(key_lo, "key_lo", torch.int32, 1, dev)
        _need(key_hi, "key_hi", torch.int32, 1, dev)
        if key_lo.shape[0] != Tq or key_hi.shape[0] != Tq:
            raise ValueError(f"key_lo and key_hi must have Tq={Tq} entries")
        if validate:
            cu = cu_seqlens_q.cpu()
            lens = seq_lens_k.cpu()
            row_len = torch.repeat_interleave(lens, (cu[1:] - cu[:-1]).long())
            lo_h, hi_h = key_lo.cpu(), key_hi.cpu()
            if bool((lo_h < 0).any()) or bool((hi_h > row_len).any()):
                raise ValueError("key ranges must lie in [0, seq_lens_k] of their sequence")
        lo_ptr, hi_ptr = key_lo.data_ptr(), key_hi.data_ptr()
    bm_ptr, bm_q, bm_k = None, 0, 0
    if block_map is not None:
        _need(block_map, "block_map", torch.uint8, 3, dev)
        if block_map.shape[0] != B:
            raise ValueError(f"block_map must be [B={B}, query blocks, key blocks]")
        bm_ptr, bm_q, bm_k = block_map.data_ptr(), block_map.shape[1], block_map.shape[2]
    ev0, ev1 = _events(kernel_events)
    general = (bool(window_left) or alibi_ptr is not None or scales is not None
               or ev0 is not None or lo_ptr is not None or persistent or bm_ptr is not None)
    if general and split is None:
        split = (1, None)                         # the plain launch, through prefill_ex
    if split is not None:
        num_splits, workspace = split
        need = int(lib.paged_attn_prefill_workspace_bytes(B, Tq, int(max_q_len), Hq, D,
                                                          num_splits))
        if workspace is not None:
            _need(workspace, "workspace", torch.uint8, 1, dev)
        elif need:
            workspace = _internal(torch.empty(need, dtype=torch.uint8, device=dev), stream)
        ws_bytes = 0 if workspace is None else workspace.numel()
    with torch.cuda.device(dev):
        if split is None:
            _check(lib.paged_attn_prefill_varlen(*args, _stream(stream)))
        elif general:
            ks, vs = _pool_scales(scales) if scales is not None else (1.0, 1.0)
            ksp = vsp = None
            if isinstance(scales, _PageScales):
                ksp, vsp = scales.check(k_pool.shape, dev)
            opts = _lib.PrefillOpts(1 if causal else 0, window_left, num_splits, alibi_ptr,
                                    0 if scales is None else 1, ks, vs, ev0, ev1, lo_ptr, hi_ptr,
                                    ksp, vsp, 1 if persistent else 0, bm_ptr, bm_q, bm_k)
            _check(lib.paged_attn_prefill_ex(*args[:-1], ctypes.byref(opts), _ptr(workspace),
                                             ws_bytes, _stream(stream)))
        else:
            _check(lib.paged_attn_prefill_varlen_splitk(*args, num_splits, _ptr(workspace),
                                                        ws_bytes, _stream(stream)))
    return (out, lse) if return_lse else out


def mixed_workspace_bytes(Hq: int, Hkv: int, D: int, prefill=None, decode=None,
                          fp8: bool = False) -> int:
    """Workspace bytes of paged_attn_mixed for the host-side sizes of its parts:
    prefill = (B, Tq, max_q_len, num_splits), decode = (B, max_seq_len, num_splits),
    either None for no such part; fp8 for FP8 pools (the decode's split rule differs)."""
    p = _lib.MixedPrefill()
    d = _lib.MixedDecode()
    if prefill is not None:
        p.B, p.Tq, p.max_q_len, p.num_splits = (int(x) for x in prefill)
    if decode is not None:
        d.B, d.max_seq_len, d.num_splits = (int(x) for x in decode)
    f = ctypes.byref(_lib.MixedFp8(1.0, 1.0, None, None)) if fp8 else None
    return int(load_library().paged_attn_mixed_workspace_bytes(ctypes.byref(p), ctypes.byref(d),
                                                               f, int(Hq), int(Hkv), int(D)))


def paged_attn_mixed(k_pool, v_pool, softmax_scale: float, prefill=None, decode=None,
                     causal: bool = True, prefill_max_q_len: Optional[int] = None,
                     prefill_num_splits: int = 0, decode_max_seq_len: Optional[int] = None,
                     decode_num_splits: int = 0, prefill_out: Optional[torch.Tensor] = None,
                     decode_out: Optional[torch.Tensor] = None,
                     prefill_lse: Optional[torch.Tensor] = None,
                     decode_lse: Optional[torch.Tensor] = None, return_lse: bool = False,
                     workspace: Optional[torch.Tensor] = None, stream=None,
                     validate: bool = False, k_scale=None, v_scale=None):
    """A step's prefill chunks and decode rows over the same bf16 pools in one kernel
    launch (then the merges of their key parts and partitions): see paged_attn_mixed
    in C.

    ``prefill`` = (q [Tq, Hq, D], cu_seqlens_q [B+1], seq_lens_k [B], block_tables), as
    paged_attn_prefill_varlen_splitk takes them; ``decode`` = (q [B, Hq, D],
    block_tables, seq_lens), as paged_attn_decode takes them; either may be None.
    ``prefill_num_splits`` <= 0 takes the library's key-part count for 256-row tiles;
    ``decode_num_splits`` <= 0 the decode's split rule.  Host-side bounds read from
    the device when omitted (a synchronisation).  Returns (prefill_out, decode_out),
    with (prefill_lse, decode_lse) after them when ``return_lse``; a missing part's
    entries are None.  Outputs and lse buffers may be passed in (``*_out``,
    ``*_lse``), as for graph capture.  With ``k_scale`` and ``v_scale`` the pools hold
    FP8 E4M3 codes under those scales (floats: one per pool; float32 tensors
    [num_pages, Hkv]: per page and KV head), as paged_attn_decode_fp8 takes them."""
    scales = None
    if k_scale is not None or v_scale is not None:
        if k_scale is None or v_scale is None:
            raise TypeError("k_scale and v_scale must both be given for FP8 pools")
        scales = _scales(k_scale, v_scale)
        _need_fp8_dtype(k_pool, "k_pool")
        _need_fp8_dtype(v_pool, "v_pool")
    else:
        _dtypes((k_pool, "k_pool", torch.bfloat16), (v_pool, "v_pool", torch.bfloat16))
    _dtypes((prefill_out, "prefill_out", torch.bfloat16),
            (decode_out, "decode_out", torch.bfloat16),
            (prefill_lse, "prefill_lse", torch.float32), (decode_lse, "decode_lse", torch.float32))
    if prefill is None and decode is None:
        raise ValueError("paged_attn_mixed needs a prefill part, a decode part or both")
    dev = (prefill or decode)[0].device
    if scales is None:
        _need(k_pool, "k_pool", torch.bfloat16, 4, dev)
        _need(v_pool, "v_pool", torch.bfloat16, 4, dev)
    else:
        _need_fp8_pool(k_pool, "k_pool", dev)
        _need_fp8_pool(v_pool, "v_pool", dev)
    P, ps, Hkv, D = k_pool.shape
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool must have the same shape")
    Hq = None
    mp = _lib.MixedPrefill()
    md = _lib.MixedDecode()
    pf_out = pf_lse = dec_out = dec_lse = None
    if prefill is not None:
        q, cu, lens, bt = prefill
        _dtypes((q, "prefill q", torch.bfloat16), (cu, "cu_seqlens_q", torch.int32),
                (lens, "seq_lens_k", torch.int32), (bt, "prefill block_tables", torch.int32))
        _need(q, "prefill q", torch.bfloat16, 3, dev)
        _need(cu, "cu_seqlens_q", torch.int32, 1, dev)
        _need(lens, "seq_lens_k", torch.int32, 1, dev)
        _need(bt, "prefill block_tables", torch.int32, 2, dev)
        Tq, Hq, Dq = q.shape
        B = lens.shape[0]
        if Dq != D:
            raise ValueError("prefill q does not match the pools' head dim")
        if cu.shape[0] != B + 1 or bt.shape[0] != B:
            raise ValueError("cu_seqlens_q must be [B+1] and block_tables [B, max_pages]")
        if prefill_max_q_len is None:
            prefill_max_q_len = int((cu[1:] - cu[:-1]).max().item()) if B else 0
        if validate:
            cu_h = cu.cpu()
            if int(cu_h[0]) != 0 or int(cu_h[-1]) != Tq or bool((cu_h[1:] < cu_h[:-1]).any()):
                raise ValueError("cu_seqlens_q must be non-decreasing from 0 to Tq")
            if B and int((cu_h[1:] - cu_h[:-1]).max()) > prefill_max_q_len:
                raise ValueError("prefill_max_q_len is below a sequence's query count")
            _validate_tables(bt, lens, P, ps)
        pf_out = prefill_out
        if pf_out is None:
            pf_out = _internal(torch.empty((Tq, Hq, D), dtype=torch.bfloat16, device=dev), stream)
        else:
            _need(pf_out, "prefill_out", torch.bfloat16, 3, dev)
            if tuple(pf_out.shape) != (Tq, Hq, D):
                raise ValueError("prefill_out must be [Tq, Hq, D]")
        pf_lse = prefill_lse
        if pf_lse is not None:
            _need(pf_lse, "prefill_lse", torch.float32, 2, dev)
            if tuple(pf_lse.shape) != (Tq, Hq):
                raise ValueError("prefill_lse must be [Tq, Hq]")
        elif return_lse:
            pf_lse = _internal(torch.empty((Tq, Hq), dtype=torch.float32, device=dev), stream)
        mp.out, mp.lse_out, mp.q = _ptr(pf_out), _ptr(pf_lse), _ptr(q)
        mp.cu_seqlens_q, mp.seq_lens_k, mp.block_tables = _ptr(cu), _ptr(lens), _ptr(bt)
        mp.B, mp.Tq, mp.max_q_len, mp.max_pages = B, Tq, int(prefill_max_q_len), bt.shape[1]
        mp.causal, mp.num_splits = 1 if causal else 0, int(prefill_num_splits)
    if decode is not None:
        q, bt, lens = decode
        _dtypes((q, "decode q", torch.bfloat16), (bt, "decode block_tables", torch.int32),
                (lens, "seq_lens", torch.int32))
        _need(q, "decode q", torch.bfloat16, 3, dev)
        _need(bt, "decode block_tables", torch.int32, 2, dev)
        _need(lens, "seq_lens", torch.int32, 1, dev)
        B, Hq_d, Dq = q.shape
        if Hq is not None and Hq_d != Hq:
            raise ValueError("the prefill and decode parts must have the same Hq")
        Hq = Hq_d
        if Dq != D:
            raise ValueError("decode q does not match the pools' head dim")
        if lens.shape[0] != B or bt.shape[0] != B:
            raise ValueError("seq_lens must be [B] and block_tables [B, max_pages]")
        if decode_max_seq_len is None:
            decode_max_seq_len = int(lens.max().item()) if B else 0
        if validate:
            _validate_tables(bt, lens, P, ps)
            if B and int(lens.max().item()) > decode_max_seq_len:
                raise ValueError("decode_max_seq_len is below a sequence length")
        dec_out = decode_out
        if dec_out is None:
            dec_out = _internal(torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev), stream)
        else:
            _need(dec_out, "decode_out", torch.bfloat16, 3, dev)
            if tuple(dec_out.shape) != (B, Hq, D):
                raise ValueError("decode_out must be [B, Hq, D]")
        dec_lse = decode_lse
        if dec_lse is not None:
            _need(dec_lse, "decode_lse", torch.float32, 2, dev)
            if tuple(dec_lse.shape) != (B, Hq):
                raise ValueError("decode_lse must be [B, Hq]")
        elif return_lse:
            dec_lse = _internal(torch.empty((B, Hq), dtype=torch.float32, device=dev), stream)
        md.out, md.lse_out, md.q = _ptr(dec_out), _ptr(dec_lse), _ptr(q)
        md.block_tables, md.seq_lens = _ptr(bt), _ptr(lens)
        md.B, md.max_pages, md.max_seq_len = B, bt.shape[1], int(decode_max_seq_len)
        md.num_splits = int(decode_num_splits)
    lib = load_library()
    f8 = None
    if scales is not None:
        ksp = vsp = None
        if isinstance(scales, _PageScales):
            ksp, vsp = scales.check(k_pool.shape, dev)
        f8 = ctypes.byref(_lib.MixedFp8(*_pool_scales(scales), ksp, vsp))
    need = int(lib.paged_attn_mixed_workspace_bytes(ctypes.byref(mp), ctypes.byref(md), f8, Hq,
                                                    Hkv, D))
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1, dev)
    elif need:
        workspace = _internal(torch.empty(need, dtype=torch.uint8, device=dev), stream)
    ws_bytes = 0 if workspace is None else workspace.numel()
    with torch.cuda.device(dev):
        _check(lib.paged_attn_mixed(ctypes.byref(mp), ctypes.byref(md), f8, _ptr(k_pool),
                                    _ptr(v_pool), P, ps, Hq, Hkv, D, float(softmax_scale),
                                    _ptr(workspace), ws_bytes, _stream(stream)))
    if return_lse:
        return pf_out, dec_out, pf_lse, dec_lse
    return pf_out, dec_out
