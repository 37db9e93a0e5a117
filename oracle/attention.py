"""Plain float64 attention over a paged KV cache (CPU, NumPy).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  This module is slow
on purpose: it gathers each sequence's pages into a dense array and
materialises the full score matrix for every query head, which is exactly
the computation a tiled kernel avoids.

Conventions shared by every function:

* bf16 tensors arrive as ``uint16`` bit patterns (or already as floats) and
  are widened exactly to float64;
* ``q``        : [T, Hq, D]   query rows of all sequences, packed;
* pools        : [P, page_size, Hkv, D]   key / value pages;
* ``block_tables`` : [B, max_pages] int, entry = physical page id;
* ``seq_lens_k``   : [B] number of keys each sequence attends to;
* ``cu_seqlens_q`` : [B+1] prefix sums of the query rows per sequence.

Readings of points the pages leave open (each is restated where used):

R1  GQA: query head h reads key/value head ``h // (Hq // Hkv)``.
R2  Causal alignment: a chunk of q_len queries sits at the END of its
    sequence, so query i has absolute position ``L - q_len + i`` and may see
    keys ``j <= L - q_len + i`` (the FlexAttention mask ``q_idx >= kv_idx`` of
    "The Stack Below the Stack (Part 2)", section 5, in absolute positions).
R3  A row with no visible key returns O = 0 and lse = -inf ("Test the kernel
    at three levels": a fully masked row must give a defined value, not the
    NaN of a zero denominator).
R4  Sliding window: the pages list sliding windows among the masks a serving
    backend must support ("8. Kernels and Attention Backends", "Attention is an
    I/O problem"; FlexAttention mask functions in "The Stack Below the Stack
    (Part 2)", section 5) without fixing the predicate.  With window w > 0 a
    query at absolute position p sees key j only if p - w < j (its last w
    positions, itself included), on top of the causal condition when causal;
    without causal only this lower bound applies.  w = 0 means no window.
R5  ALiBi: "The Stack Below the Stack (Part 2)", section 5, names ALiBi among the
    score modifications a FlexAttention function expresses, without a formula.
    Reading: with one slope per query head (given by the caller), the score of
    query h at absolute position p against key j becomes
    scale * q . k + slope_h * (j - p), i.e. a linear penalty on the distance to
    earlier keys for positive slopes.  No slopes means no bias.
R6  Document masks: the same section names document masking among the mask
    functions (a query sees only keys of its own document; several documents
    packed into one sequence) without fixing a representation.  Reading: the
    documents of a sequence are contiguous runs of positions, and the caller
    gives every query row the half-open range [key_lo, key_hi) of key
    positions of its own document; the row sees key j only if
    key_lo <= j < key_hi, on top of the causal bound and the window.  No
    ranges means every row's range is the whole sequence.
R7  Mask functions: the same section shows a mask written as a predicate of
    (sequence b, head h, query index, key index) and compiled with
    create_block_mask, which records per (query block, key block) whether the
    block needs the predicate at all.  Reading: a general mask is such a predicate
    with the query index counted within the sequence's query run (row i of the
    run, 0-based) and the key index within the sequence; the row sees key j only
    if the predicate holds, on top of the causal bound, the window and the
    document range.  A block map is the block form of a predicate that is
    constant on blocks: entry [b][i // 64][j // 64] (nonzero: visible); entries
    outside the map count as zero.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "gather_sequence_kv",
    "attend_rows",
    "attention_ref",
    "attention_rows_ref",
    "block_map_mask",
    "softmax_probs_ref",
    "tiled_attend_rows",
    "split_partials_ref",
    "merge_ref",
    "kv_write_ref",
]


def bf16_bits_to_f64(x) -> np.ndarray:
    """Widen bf16 values, given as uint16 bit patterns, to float64 exactly.

    A bf16 value is the upper half of an IEEE binary32; shifting the 16 bits
    into the top of a 32-bit word and reinterpreting gives the same number.
    Float input is passed through as float64.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype == np.int16:
        return bf16_bits_to_f64(x.view(np.uint16))
    return x.astype(np.float64)


def gather_sequence_kv(pool, table_row, seq_len: int, page_size: int) -> np.ndarray:
    """Logical keys (or values) 0..seq_len-1 of one sequence, [seq_len, Hkv, D].

    Paged KV (Ion post, "IonAttention in One Paragraph"; the inference guide,
    chapter 8 intro: KV blocks scattered through memory): logical key j lives
    in page ``table_row[j // page_size]`` at row ``j % page_size``.  Only the
    first ceil(seq_len / page_size) table entries are read.
    """
    pool = bf16_bits_to_f64(pool)
    if seq_len == 0:
        return np.zeros((0,) + pool.shape[2:], dtype=np.float64)
    n_pages = -(-seq_len // page_size)
    pages = np.asarray(table_row[:n_pages], dtype=np.int64)
    if pages.min() < 0 or pages.max() >= pool.shape[0]:
        raise ValueError("block table references a page outside the pool")
    dense = pool[pages].reshape(n_pages * page_size, *pool.shape[2:])
    return dense[:seq_len]


def attend_rows(q_rows, k, v, scale: float, visible, first=None, slope: float = 0.0,
                pos=None, allowed=None):
    """Plain softmax attention for a set of query rows against one key head.

    ``q_rows`` [n, D], ``k``/``v`` [L, D], ``visible`` [n] = number of leading
    keys each row may see; ``first`` [n] (optional) = index of the first key
    each row may see (R4; default 0); ``slope`` with ``pos`` [n] (the rows'
    absolute positions) adds slope * (j - pos_i) to every score (R5).  Returns
    (O [n, D], lse [n]) in float64.  ``allowed`` [n, L] (optional, boolean): a
    general mask on top of the others (R7); False hides the key.

    This is the definition the tiled method must reproduce exactly ("8.
    Kernels and Attention Backends", "Attention is an I/O problem": scores
    between queries and keys, a softmax, then a product with the values):
    the full score matrix is materialised, masked keys get -inf, and the
    row-wise softmax multiplies V.  lse is the natural-log log-sum-exp of
    the visible scores.  A row that sees no key gives O = 0, lse = -inf (R3).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, L = q_rows.shape[0], k.shape[0]
    visible = np.asarray(visible, dtype=np.int64).reshape(n)
    out = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    if n == 0 or L == 0:
        return out, lse
    s = scale * (q_rows @ k.T)                                   # [n, L]
    if slope != 0.0:
        pos = np.asarray(pos, dtype=np.float64).reshape(n)
        s = s + float(slope) * (np.arange(L, dtype=np.float64)[None, :] - pos[:, None])
    mask = np.arange(L)[None, :] >= visible[:, None]
    if first is not None:
        first = np.asarray(first, dtype=np.int64).reshape(n)
        mask |= np.arange(L)[None, :] < first[:, None]
    if allowed is not None:
        mask |= ~np.broadcast_to(np.asarray(allowed, dtype=bool), (n, L))
    s = np.where(mask, -np.inf, s)
    m = s.max(axis=1)
    live = np.isfinite(m)
    if not live.any():
        return out, lse
    p = np.exp(s[live] - m[live, None])
    l = p.sum(axis=1)
    out[live] = (p @ v) / l[:, None]
    lse[live] = m[live] + np.log(l)
    return out, lse


def _visible_counts(seq_len: int, q_len: int, causal: bool) -> np.ndarray:
    """Keys visible to each of the q_len rows of a sequence with seq_len keys.

    Causal (R2): row i sits at absolute position seq_len - q_len + i and sees
    keys j <= that position, i.e. ``seq_len - q_len + i + 1`` keys (clipped to
    [0, seq_len]).  Non-causal: every row sees all seq_len keys.
    """
    if not causal:
        return np.full(q_len, seq_len, dtype=np.int64)
    vis = seq_len - q_len + np.arange(q_len, dtype=np.int64) + 1
    return np.clip(vis, 0, seq_len)


def _first_visible(seq_len: int, q_len: int, window: int) -> np.ndarray:
    """Index of the first key each of the q_len rows may see under a sliding
    window (R4): row i at absolute position p = seq_len - q_len + i sees keys
    j > p - window, so the first is max(0, p - window + 1); 0 without a window."""
    if window <= 0:
        return np.zeros(q_len, dtype=np.int64)
    pos = seq_len - q_len + np.arange(q_len, dtype=np.int64)
    return np.maximum(0, pos - window + 1)


def _document_bounds(vis, first, key_ranges, t0, t1):
    """Per-row key bounds with the document ranges of R6 applied: a row sees keys
    first_i <= j < vis_i, narrowed to its own [key_lo, key_hi)."""
    if key_ranges is None:
        return vis, first
    lo = np.asarray(key_ranges[0], dtype=np.int64)[t0:t1]
    hi = np.asarray(key_ranges[1], dtype=np.int64)[t0:t1]
    return np.minimum(vis, hi), np.maximum(first, lo)


def block_map_mask(block_map, block: int = 64):
    """The predicate of a block map (R7): ``block_map`` [B, QB, KB], entry
    [b][i // block][j // block] nonzero when query row i (of the sequence's query
    run) may see key j; entries outside the map count as zero."""
    bm = np.asarray(block_map)
    if bm.ndim != 3:
        raise ValueError("block_map must be [B, query blocks, key blocks]")

    def pred(b, h, q_idx, kv_idx):
        qb = np.asarray(q_idx) // block
        kb = np.asarray(kv_idx) // block
        qb, kb = np.broadcast_arrays(qb, kb)
        inside = (qb < bm.shape[1]) & (kb < bm.shape[2])
        out = np.zeros(qb.shape, dtype=bool)
        out[inside] = bm[b][qb[inside], kb[inside]] != 0
        return out
    return pred


def _allowed(mask_fn, b, h, rows, L):
    """[len(rows), L] boolean of a predicate (R7) for the given query indices of one
    sequence's query run (all n of them when ``rows`` is an int n) and its L keys."""
    if mask_fn is None:
        return None
    qi = (np.arange(rows) if np.isscalar(rows) else np.asarray(rows))[:, None]
    kj = np.arange(L)[None, :]
    return np.broadcast_to(np.asarray(mask_fn(b, h, qi, kj), dtype=bool), (qi.shape[0], L))


def attention_ref(q, k_pool, v_pool, block_tables, seq_lens_k, cu_seqlens_q,
                  scale: float, causal: bool, page_size: int, window: int = 0, alibi=None,
                  key_ranges=None, mask_fn=None):
    """Exact attention of every query row; returns (O [T, Hq, D], lse [T, Hq]).

    ``key_ranges`` = (key_lo [T], key_hi [T]) restricts each query row to the
    keys of its own document (R6).  ``mask_fn(b, h, q_idx, kv_idx)`` (broadcasting
    over index arrays) is a general mask on top (R7); :func:`block_map_mask` makes
    one from a block map.

    Streams one (sequence, key head) at a time so that memory stays bounded
    by one sequence's score matrix per query head -- the N^2 b warning of
    "The Stack Below the Stack (Part 2)", section 2.1, is why the oracle
    never materialises scores for the whole batch at once.
    """
    q = bf16_bits_to_f64(q)
    T, Hq, D = q.shape
    Hkv = np.asarray(k_pool).shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    out = np.zeros((T, Hq, D), dtype=np.float64)
    lse = np.full((T, Hq), -np.inf, dtype=np.float64)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    lens = np.asarray(seq_lens_k, dtype=np.int64)
    for b in range(lens.shape[0]):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        if t1 == t0:
            continue
        L = int(lens[b])
        kb = gather_sequence_kv(k_pool, block_tables[b], L, page_size)
        vb = gather_sequence_kv(v_pool, block_tables[b], L, page_size)
        vis = _visible_counts(L, t1 - t0, causal)
        first = _first_visible(L, t1 - t0, window)
        vis, first = _document_bounds(vis, first, key_ranges, t0, t1)      # R6
        pos = L - (t1 - t0) + np.arange(t1 - t0)                        # R2
        for h in range(Hq):
            kvh = h // G                                                # R1
            slope = 0.0 if alibi is None else float(alibi[h])          # R5
            o, ls = attend_rows(q[t0:t1, h], kb[:, kvh], vb[:, kvh], scale, vis, first,
                                slope, pos, _allowed(mask_fn, b, h, t1 - t0, L))   # R7
            out[t0:t1, h] = o
            lse[t0:t1, h] = ls
    return out, lse


def attention_rows_ref(q, k_pool, v_pool, block_tables, seq_lens_k, cu_seqlens_q,
                       scale: float, causal: bool, page_size: int, rows, window: int = 0,
                       alibi=None, key_ranges=None, mask_fn=None):
    """Same as :func:`attention_ref` for selected (token, head) pairs only.

    Used at full workload sizes, where the oracle computes sampled outputs one
    by one.  Returns (O [n, D], lse [n]) in the order of ``rows``.
    """
    q = bf16_bits_to_f64(q)
    Hq, D = q.shape[1], q.shape[2]
    Hkv = np.asarray(k_pool).shape[2]
    G = Hq // Hkv
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    lens = np.asarray(seq_lens_k, dtype=np.int64)
    rows = [(int(t), int(h)) for t, h in rows]
    out = np.zeros((len(rows), D), dtype=np.float64)
    lse = np.full(len(rows), -np.inf, dtype=np.float64)
    by_seq = {}
    for i, (t, h) in enumerate(rows):
        b = int(np.searchsorted(cu, t, side="right") - 1)
        by_seq.setdefault(b, []).append((i, t, h))
    for b, items in by_seq.items():
        L = int(lens[b])
        q_len = int(cu[b + 1] - cu[b])
        vis_all = _visible_counts(L, q_len, causal)
        first_all = _first_visible(L, q_len, window)
        vis_all, first_all = _document_bounds(vis_all, first_all, key_ranges, int(cu[b]),
                                              int(cu[b + 1]))                   # R6
        kb = gather_sequence_kv(k_pool, block_tables[b], L, page_size)
        vb = gather_sequence_kv(v_pool, block_tables[b], L, page_size)
        for i, t, h in items:
            kvh = h // G
            i0 = t - int(cu[b])
            slope = 0.0 if alibi is None else float(alibi[h])
            o, ls = attend_rows(q[t:t + 1, h], kb[:, kvh], vb[:, kvh], scale,
                                vis_all[i0:i0 + 1], first_all[i0:i0 + 1], slope,
                                [L - q_len + i0], _allowed(mask_fn, b, h, [i0], L))
            out[i], lse[i] = o[0], ls[0]
    return out, lse


def softmax_probs_ref(q_rows, k, scale: float, visible) -> np.ndarray:
    """The attention probabilities P [n, L] that :func:`attend_rows` applies.

    Exposed so that tests can check the softmax itself (rows sum to one,
    masked keys get exactly zero).  A row with no visible key is all zeros.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n, L = q_rows.shape[0], k.shape[0]
    visible = np.asarray(visible, dtype=np.int64).reshape(n)
    s = scale * (q_rows @ k.T)
    s = np.where(np.arange(L)[None, :] >= visible[:, None], -np.inf, s)
    p = np.zeros_like(s)
    m = s.max(axis=1) if L else np.full(n, -np.inf)
    for i in range(n):
        if np.isfinite(m[i]):
            e = np.exp(s[i] - m[i])
            p[i] = e / e.sum()
    return p


def tiled_attend_rows(q_rows, k, v, scale: float, visible, tile: int):
    """Online-softmax attention walking the keys one tile at a time.

    Follows the running max / running sum description of "The Stack Below
    the Stack (Part 2)", section 2.1 (and "8. Kernels and Attention
    Backends", "Attention is an I/O problem"): for each tile the running
    maximum m is raised to cover the tile's scores, everything accumulated
    so far (the sum of exponentials l and the value accumulator) is rescaled
    by exp(m_old - m_new), and the tile's exponentials are added.  At the end
    O = acc / l and lse = m + ln l.  It must equal :func:`attend_rows`
    exactly up to rounding; the tests check that.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, L, D = q_rows.shape[0], k.shape[0], v.shape[1]
    visible = np.asarray(visible, dtype=np.int64).reshape(n)
    out = np.zeros((n, D))
    lse = np.full(n, -np.inf)
    for i in range(n):
        m, l, acc = -np.inf, 0.0, np.zeros(D)
        for j0 in range(0, L, tile):
            j1 = min(j0 + tile, L)
            s = scale * (k[j0:j1] @ q_rows[i])
            s = np.where(np.arange(j0, j1) >= visible[i], -np.inf, s)
            m_new = max(m, s.max())
            if m_new == -np.inf:          # nothing visible yet: state unchanged
                continue
            alpha = math.exp(m - m_new) if m != -np.inf else 0.0
            p = np.exp(s - m_new)
            l = alpha * l + p.sum()
            acc = alpha * acc + p @ v[j0:j1]
            m = m_new
        if l > 0.0:
            out[i] = acc / l
            lse[i] = m + math.log(l)
    return out, lse


def split_partials_ref(q_row, k, v, scale: float, visible: int, bounds):
    """Per-chunk partial results of Flash-Decoding for one query row.

    "The Stack Below the Stack (Part 2)", section 2.2: the KV sequence is cut
    into chunks along its length and each chunk yields its own normalised
    partial output plus a local log-sum-exp.  ``bounds`` lists the chunk edges
    [b0=0, b1, ..., bC=L].  A chunk with no visible key yields O_c = 0 and
    lse_c = -inf (R3).  Returns (O_c [C, D], lse_c [C]).
    """
    q_row = np.asarray(q_row, dtype=np.float64).reshape(1, -1)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    C = len(bounds) - 1
    o_c = np.zeros((C, v.shape[1]))
    lse_c = np.full(C, -np.inf)
    for c in range(C):
        a, b = int(bounds[c]), int(bounds[c + 1])
        vis = max(0, min(visible, b) - a)
        o, ls = attend_rows(q_row, k[a:b], v[a:b], scale, [vis])
        o_c[c], lse_c[c] = o[0], ls[0]
    return o_c, lse_c


def merge_ref(o_c, lse_c):
    """Combine chunk partials into the exact result (Flash-Decoding's reduce).

    "The Stack Below the Stack (Part 2)", section 2.2, step 3: the local
    log-sum-exps reweight the chunks' normalised outputs,
    lse = ln sum_c exp(lse_c) and O = sum_c exp(lse_c - lse) O_c.  Works on
    the last two axes: o_c [..., C, D], lse_c [..., C].  If every chunk is
    empty the result is O = 0, lse = -inf (R3).
    """
    o_c = np.asarray(o_c, dtype=np.float64)
    lse_c = np.asarray(lse_c, dtype=np.float64)
    m = lse_c.max(axis=-1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_c - m_safe)                        # exp(-inf) = 0 for empty chunks
    tot = w.sum(axis=-1, keepdims=True)
    tot_safe = np.where(empty, 1.0, tot)
    out = (w[..., None] * o_c).sum(axis=-2) / tot_safe
    lse = np.where(empty, -np.inf, m_safe + np.log(tot_safe))[..., 0]
    out = np.where(empty, 0.0, out)
    return out, lse


def kv_write_ref(k_pool, v_pool, k_new, v_new, cu_new, start_pos, block_tables,
                 page_size: int):
    """Write new tokens' keys and values into their pages; returns new pools.

    Eager KV writeback ("Inside Ion", "IonAttention in One Paragraph"; the
    KV-cache insertion fusions of "The Stack Below the Stack (Part 2)",
    section 2.1): new token t of sequence b has logical position
    ``start_pos[b] + (t - cu_new[b])`` and lands in page
    ``block_tables[b][pos // page_size]`` at row ``pos % page_size``, all heads
    at once.  The pools are copied, never modified in place; values are
    moved as raw bits (no arithmetic).
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    cu = np.asarray(cu_new, dtype=np.int64)
    for b in range(len(cu) - 1):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        if t1 == t0:
            continue
        pos = int(start_pos[b]) + np.arange(t1 - t0)
        pages = np.asarray(block_tables[b], dtype=np.int64)[pos // page_size]
        if pages.min() < 0 or pages.max() >= k_out.shape[0]:
            raise ValueError("write targets a page outside the pool")
        slots = pos % page_size
        k_out[pages, slots] = np.asarray(k_new)[t0:t1]
        v_out[pages, slots] = np.asarray(v_new)[t0:t1]
    return k_out, v_out
