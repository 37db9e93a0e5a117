"""Seeded synthetic inputs for paged-KV attention, shared by tests and bench.

This module draws random numbers and lays them out as a paged KV cache; it
holds none of the attention arithmetic.  Both the HIP library and the
float64 oracle consume what it produces, and it imports neither.

Layout of a case (the problem statement of the source pages: queries
[tokens, Hq, D], key/value page pools [pages, page_size, Hkv, D],
per-sequence block tables and lengths, GQA ratio, softmax scale, causal):

* ``q``            [T, Hq, D] bf16, packed query rows of all sequences;
* ``k_pool``/``v_pool`` [P, page_size, Hkv, D] bf16, the cache BEFORE any
  ``kv_page_write`` of the case's new tokens;
* ``block_tables`` [B, max_pages] int32, a seeded permutation of the pool
  handed out in sequence order; entries past a sequence's last page are -1;
* ``seq_lens_k``   [B] int32, keys attended (history + new tokens);
* ``cu_seqlens_q`` [B+1] int32;
* ``k_new``/``v_new`` [Tn, Hkv, D], ``cu_new`` [B+1], ``start_pos`` [B]:
  tokens that ``kv_page_write`` must place before attention (None when the
  pools already hold every key).

Poison, so that a wrong gather cannot go unnoticed:

* pages no table references are filled with bf16 NaN;
* slots past a sequence's last key in its last page hold +-3e4 (finite);
* slots that ``kv_page_write`` must fill start as NaN.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

__all__ = ["PagedCase", "make_case", "make_config", "config_shape", "CONFIGS",
           "CONFIG_ORDER", "bits", "units", "random_e4m3_codes", "document_ranges"]

BF16_NAN_BITS = 0x7FC0
TAIL_POISON = 3.0e4


@dataclass
class PagedCase:
    name: str
    Hq: int
    Hkv: int
    D: int
    page_size: int
    scale: float
    causal: bool
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    block_tables: torch.Tensor
    seq_lens_k: torch.Tensor
    cu_seqlens_q: torch.Tensor
    hist_lens: List[int]
    q_lens: List[int]
    k_new: Optional[torch.Tensor] = None
    v_new: Optional[torch.Tensor] = None
    cu_new: Optional[torch.Tensor] = None
    start_pos: Optional[torch.Tensor] = None
    num_splits: int = 0
    window: int = 0                               # sliding window (0: none)
    meta: dict = field(default_factory=dict)
    host_seq_lens: Optional[List[int]] = None     # keys attended, kept on the host

    @property
    def B(self) -> int:
        return int(self.seq_lens_k.shape[0])

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def seq_lens(self) -> List[int]:
        if self.host_seq_lens is not None:
            return list(self.host_seq_lens)
        return [int(x) for x in self.seq_lens_k.cpu().tolist()]

    @property
    def max_seq_len(self) -> int:
        return max(self.seq_lens) if self.B else 0

    @property
    def max_q_len(self) -> int:
        return max(self.q_lens) if self.q_lens else 0

    def to(self, device) -> "PagedCase":
        out = PagedCase(**{k: getattr(self, k) for k in self.__dataclass_fields__})
        for k in ("q", "k_pool", "v_pool", "block_tables", "seq_lens_k", "cu_seqlens_q",
                  "k_new", "v_new", "cu_new", "start_pos"):
            t = getattr(self, k)
            if t is not None:
                setattr(out, k, t.to(device))
        return out


def bits(t: torch.Tensor) -> np.ndarray:
    """A bf16 tensor's raw bits as a host uint16 array (for the oracle)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _randn_bf16(shape, std, gen, device, chunk_rows=None):
    """Normal(0, std) values rounded to bf16 (round-to-nearest-even)."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    if chunk_rows is None or shape[0] <= chunk_rows:
        out.copy_(torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std)
        return out
    for r in range(0, shape[0], chunk_rows):
        n = min(chunk_rows, shape[0] - r)
        out[r:r + n].copy_(torch.randn((n,) + tuple(shape[1:]), generator=gen, device=device,
                                       dtype=torch.float32) * std)
    return out


def random_e4m3_codes(shape, seed: int, device="cpu", exp_lo: int = 4,
                      exp_hi: int = 10) -> torch.Tensor:
    """Seeded random bytes shaped like FP8 E4M3 codes, as uint8: a random sign bit,
    a 4-bit exponent field drawn uniformly from [exp_lo, exp_hi] and a random 3-bit
    mantissa field.  With the default window every code is a finite normal number
    and none is a NaN code (those need the exponent field 15).  Used for FP8 pools
    too large to build from float data on the host."""
    if not (0 <= exp_lo <= exp_hi <= 14):
        raise ValueError("exponent window must lie in [0, 14]")
    gen = torch.Generator(device=device).manual_seed(seed)
    e = torch.randint(exp_lo, exp_hi + 1, shape, generator=gen, device=device, dtype=torch.int32)
    m = torch.randint(0, 8, shape, generator=gen, device=device, dtype=torch.int32)
    s = torch.randint(0, 2, shape, generator=gen, device=device, dtype=torch.int32)
    return ((s << 7) | (e << 3) | m).to(torch.uint8)


def make_case(name, seq_lens=None, Hq=8, Hkv=2, D=64, page_size=16, num_pages=None,
              seed=0, q_lens=None, hist_lens=None, causal=False, write_new=False,
              std_q=1.0, std_kv=1.0, scale=None, device="cpu", num_splits=0,
              max_pages=None, permute=True, window=0) -> PagedCase:
    """Build one seeded case.

    Two shapes of case:

    * decode-style (``write_new=False``): ``seq_lens[b]`` keys already sit in
      the pools; ``q_lens[b]`` query rows per sequence (default 1).
    * write-then-attend (``write_new=True``): ``hist_lens[b]`` keys already sit
      in the pools and ``q_lens[b]`` new tokens arrive with their own K/V,
      which ``kv_page_write`` places at positions hist..hist+q_len-1 before
      attention; ``seq_lens_k = hist + q_len``.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    if write_new:
        hist = [int(x) for x in hist_lens]
        ql = [int(x) for x in q_lens]
        total = [h + n for h, n in zip(hist, ql)]
    else:
        total = [int(x) for x in seq_lens]
        ql = [1] * len(total) if q_lens is None else [int(x) for x in q_lens]
        hist = [t - n for t, n in zip(total, ql)]
    B = len(total)
    n_pages = [-(-L // page_size) for L in total]
    used = sum(n_pages)
    if num_pages is None:
        num_pages = max(used, 1)
    if used > num_pages:
        raise ValueError(f"{used} pages needed, pool has {num_pages}")
    if max_pages is None:
        max_pages = max(max(n_pages) if n_pages else 1, 1)
    perm = rng.permutation(num_pages) if permute else np.arange(num_pages)
    bt = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :n_pages[b]] = perm[off:off + n_pages[b]]
        off += n_pages[b]
    referenced = perm[:used]

    shape = (num_pages, page_size, Hkv, D)
    chunk = max(1, (1 << 26) // (page_size * Hkv * D))
    k_pool = _randn_bf16(shape, std_kv, gen, device, chunk)
    v_pool = _randn_bf16(shape, std_kv, gen, device, chunk)

    # poison: unreferenced pages -> NaN
    unref = np.setdiff1d(np.arange(num_pages), referenced)
    nan = torch.tensor(BF16_NAN_BITS, dtype=torch.int16).view(torch.bfloat16).item()
    if unref.size:
        idx = torch.as_tensor(unref, device=device, dtype=torch.long)
        k_pool[idx] = nan
        v_pool[idx] = nan
    # poison: slots past the last key of each sequence's last page -> +-3e4
    for b in range(B):
        L = total[b]
        if L % page_size and n_pages[b]:
            page = int(bt[b, n_pages[b] - 1])
            k_pool[page, L % page_size:] = TAIL_POISON
            v_pool[page, L % page_size:] = -TAIL_POISON
    T = sum(ql)
    q = _randn_bf16((max(T, 0), Hq, D), std_q, gen, device)
    cu_q = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)

    k_new = v_new = cu_new = start_pos = None
    if write_new:
        k_new = _randn_bf16((T, Hkv, D), std_kv, gen, device)
        v_new = _randn_bf16((T, Hkv, D), std_kv, gen, device)
        # the slots the writer must fill start as NaN
        for b in range(B):
            if ql[b] == 0:
                continue
            pos = np.arange(hist[b], total[b])
            pages = torch.as_tensor(bt[b, pos // page_size].astype(np.int64), device=device)
            slots = torch.as_tensor(pos % page_size, device=device, dtype=torch.long)
            k_pool[pages, slots] = nan
            v_pool[pages, slots] = nan
        cu_new = torch.as_tensor(cu_q, device=device)
        start_pos = torch.as_tensor(np.asarray(hist, dtype=np.int32), device=device)

    return PagedCase(
        name=name, Hq=Hq, Hkv=Hkv, D=D, page_size=page_size,
        scale=(1.0 / math.sqrt(D)) if scale is None else float(scale), causal=causal,
        q=q, k_pool=k_pool, v_pool=v_pool,
        block_tables=torch.as_tensor(bt, device=device),
        seq_lens_k=torch.as_tensor(np.asarray(total, dtype=np.int32), device=device),
        cu_seqlens_q=torch.as_tensor(cu_q, device=device),
        hist_lens=hist, q_lens=ql, k_new=k_new, v_new=v_new, cu_new=cu_new,
        start_pos=start_pos, num_splits=num_splits, window=int(window),
        meta=dict(seed=seed, std_q=std_q, std_kv=std_kv), host_seq_lens=list(total),
    )


def document_ranges(seq_lens, q_lens, docs_per_seq, seed: int):
    """Seeded packed-document layout: every sequence's positions 0 .. L-1 are cut
    into up to docs_per_seq contiguous documents at random boundaries, and each query
    row (the last q_len positions of its sequence) gets the half-open key range
    [key_lo, key_hi) of the document holding its position.  Returns host int32
    arrays (key_lo, key_hi) of length sum(q_lens).  Structure only: no attention
    arithmetic."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lo_all, hi_all = [], []
    for L, n in zip(seq_lens, q_lens):
        L, n = int(L), int(n)
        k = max(1, min(int(docs_per_seq), L)) if L > 0 else 1
        cuts = np.sort(rng.choice(np.arange(1, L), size=k - 1, replace=False)) if k > 1 \
            else np.zeros(0, dtype=np.int64)
        starts = np.concatenate([[0], cuts]).astype(np.int64)
        ends = np.concatenate([cuts, [max(L, 0)]]).astype(np.int64)
        for i in range(n):
            p = L - n + i                       # the row's absolute position
            d = int(np.searchsorted(starts, p, side="right") - 1) if p >= 0 else -1
            if d < 0:                           # a row before the sequence's first key
                lo_all.append(0)
                hi_all.append(0)
            else:
                lo_all.append(int(starts[d]))
                hi_all.append(int(ends[d]))
    return np.asarray(lo_all, dtype=np.int32), np.asarray(hi_all, dtype=np.int32)


def local_strided_block_map(q_blocks: int, k_blocks: int, local: int = 4, stride: int = 8,
                            offset_blocks: int = 0):
    """A structured sparse mask in block form (64 x 64 blocks): query block i sees the
    key blocks within `local` blocks below its own position (i + offset_blocks) and
    every `stride`-th block before that.  uint8 [q_blocks, k_blocks]."""
    i = np.arange(q_blocks)[:, None] + offset_blocks
    j = np.arange(k_blocks)[None, :]
    return (((i - local < j) & (j <= i)) | (j % stride == 0)).astype(np.uint8)


def _mixed_lengths(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    hist = np.clip(np.rint(rng.lognormal(7.0, 1.0, size=23)), 16, 32768).astype(np.int64)
    q_lens = [512] * 5 + [1] * 18
    return [int(h) for h in hist], q_lens


# The five workloads.  Seeds are 1000 + the workload's index.
CONFIG_ORDER = ["tiny_decode", "qwen7b_decode", "mixed_ragged", "causal_prefill", "long_decode"]


def _shapes():
    """make_case arguments of every named workload (structure and sizes only)."""
    hist, ql = _mixed_lengths(1002)
    return {
        "tiny_decode": dict(seq_lens=[17, 64, 100, 255], Hq=8, Hkv=2, D=64, page_size=16,
                            num_pages=64, seed=1000, num_splits=1),
        "qwen7b_decode": dict(seq_lens=[8192] * 32, Hq=28, Hkv=4, D=128, page_size=16,
                              num_pages=16384, seed=1001),
        "mixed_ragged": dict(hist_lens=hist, q_lens=ql, write_new=True, causal=True, Hq=32,
                             Hkv=8, D=128, page_size=16, seed=1002),
        "causal_prefill": dict(hist_lens=[0] * 4, q_lens=[4096] * 4, write_new=True,
                               causal=True, Hq=32, Hkv=8, D=128, page_size=16,
                               num_pages=1024, seed=1003),
        "long_decode": dict(seq_lens=[131072] * 8, Hq=64, Hkv=8, D=128, page_size=64,
                            num_pages=16384, seed=1004, std_kv=0.5, num_splits=64),
        # one 512-token prefill chunk over a 32,768-token history (chunked prefill of a
        # long prompt): only 128 query tiles, the case key splitting is for
        "long_history_chunk": dict(hist_lens=[32768], q_lens=[512], write_new=True,
                                   causal=True, Hq=32, Hkv=8, D=128, page_size=16, seed=1005),
    }


CONFIGS = {name: (lambda device, n=name: make_case(n, device=device, **_shapes()[n]))
           for name in _shapes()}


def config_shape(name: str) -> dict:
    """The named workload's host-side structure without generating any values:
    seq_lens (keys attended), q_lens, Hq, Hkv, D, page_size."""
    a = _shapes()[name]
    if a.get("write_new"):
        ql = list(a["q_lens"])
        lens = [h + n for h, n in zip(a["hist_lens"], ql)]
    else:
        lens = list(a["seq_lens"])
        ql = [1] * len(lens) if a.get("q_lens") is None else list(a["q_lens"])
    return dict(seq_lens=lens, q_lens=ql, Hq=a["Hq"], Hkv=a["Hkv"], D=a["D"],
                page_size=a["page_size"])


def make_config(name: str, device="cpu") -> PagedCase:
    return CONFIGS[name](device)


from . import units  # noqa: E402,F401
