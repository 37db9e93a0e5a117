"""Algorithmic work units: the bytes and flops a paged-attention call must move.

These count what the method has to touch, not what a kernel happens to
touch, so that achieved GB/s and TFLOP/s measure kernel quality:

* decode bytes: every attended key and value element once per KV head (not
  per query head), plus Q, O, the block-table entries actually used and the
  lengths.  Split-K partials are overhead and are not counted.
* prefill flops: 4 * D per unmasked (query, key) pair per query head (one
  multiply-add for QK^T and one for PV).  Masked pairs are not counted.

The per-head figures that the inference guide's chapter 8, section
"Counting attention's traffic", prints are reproduced by
``kv_bytes_per_head`` and ``score_matrix_bytes``; the N^2 b intermediate of
"The Stack Below the Stack (Part 2)", section 2.1, by ``score_matrix_bytes``.
"""

from __future__ import annotations

from typing import Optional, Sequence


def kv_bytes_per_head(seq_len: int, head_dim: int, elem_bytes: int = 2) -> int:
    """Bytes of keys plus values one head streams for a sequence: 2 * L * D * b."""
    return 2 * seq_len * head_dim * elem_bytes


def score_matrix_bytes(n_q: int, n_k: int, elem_bytes: int = 2) -> int:
    """Bytes of a materialised score matrix: n_q * n_k * b (N^2 b when square)."""
    return n_q * n_k * elem_bytes


def naive_attention_traffic(seq_len: int, elem_bytes: int = 2, passes: int = 3) -> int:
    """HBM traffic of the unfused score matrix per head: written, read, read again."""
    return passes * score_matrix_bytes(seq_len, seq_len, elem_bytes)


def decode_bytes(seq_lens: Sequence[int], Hq: int, Hkv: int, D: int, page_size: int,
                 elem_bytes: int = 2, kv_elem_bytes: Optional[int] = None) -> int:
    """Algorithmic bytes of one decode call (one query row per sequence).  Q and O
    take elem_bytes per element, the K/V pools kv_elem_bytes (1 for FP8 pools;
    elem_bytes when not given)."""
    B = len(seq_lens)
    kvb = elem_bytes if kv_elem_bytes is None else kv_elem_bytes
    kv = sum(kv_bytes_per_head(L, D, kvb) * Hkv for L in seq_lens)
    q = B * Hq * D * elem_bytes
    o = B * Hq * D * elem_bytes
    tables = sum(-(-L // page_size) for L in seq_lens) * 4
    lens = B * 4
    return kv + q + o + tables + lens


def prefill_pairs(seq_lens: Sequence[int], q_lens: Sequence[int], causal: bool) -> int:
    """Unmasked (query, key) pairs per query head over a ragged batch.

    Causal rows sit at the end of their sequence: row i of a chunk of q_len
    rows over L keys sees L - q_len + i + 1 keys.
    """
    total = 0
    for L, n in zip(seq_lens, q_lens):
        if not causal:
            total += n * L
            continue
        # sum over i < n of max(0, L - n + 1 + i): an arithmetic series over
        # the rows that see at least one key
        first = L - n + 1
        skip = max(0, 1 - first)          # rows that see nothing
        rows = n - skip
        lo = first + skip
        total += rows * lo + rows * (rows - 1) // 2
    return total


def block_map_pairs(seq_lens: Sequence[int], q_lens: Sequence[int], causal: bool,
                    block_map, block: int = 64) -> int:
    """Unmasked (query, key) pairs per query head with a block map on top: row i of
    sequence b's query run sees key j only if block_map[b][i // block][j // block]
    is nonzero (entries outside the map count as zero), and the causal bound."""
    import numpy as np
    bm = np.asarray(block_map)
    total = 0
    for b, (L, n) in enumerate(zip(seq_lens, q_lens)):
        for qb in range(min(bm.shape[1], -(-n // block))):
            rows = np.arange(qb * block, min(n, qb * block + block))
            # keys each row sees: [0, L) or, causal, [0, L - n + i]
            lim = np.minimum(L, L - n + rows + 1) if causal else np.full(rows.shape, L)
            for kb in np.nonzero(bm[b, qb, :min(bm.shape[2], -(-L // block))])[0]:
                lo = kb * block
                total += int(np.clip(lim - lo, 0, block).sum())
    return total


def prefill_flops(seq_lens: Sequence[int], q_lens: Sequence[int], Hq: int, D: int,
                  causal: bool) -> int:
    """Algorithmic flops: 4 * D * Hq per unmasked (query, key) pair."""
    return 4 * D * Hq * prefill_pairs(seq_lens, q_lens, causal)


def prefill_bytes(seq_lens: Sequence[int], q_lens: Sequence[int], Hq: int, Hkv: int,
                  D: int, elem_bytes: int = 2) -> int:
    """Minimum HBM traffic of a prefill call: Q, O once, K and V once per KV head."""
    T = sum(q_lens)
    return 2 * T * Hq * D * elem_bytes + sum(kv_bytes_per_head(L, D, elem_bytes) * Hkv
                                             for L in seq_lens)


def kv_write_bytes(n_tokens: int, Hkv: int, D: int, elem_bytes: int = 2) -> int:
    """Bytes a KV page write moves: K and V rows read once and written once."""
    return 2 * 2 * n_tokens * Hkv * D * elem_bytes
