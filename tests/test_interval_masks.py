"""Masks that are one key interval per query row, given to the kernels as per-row
key ranges (key_lo / key_hi) and to the oracle as general predicates (reading R7):
a prefix-LM mask and chunked local attention."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_flashattention_amd as pa
from tests.parity import as_f64, assert_lse, assert_parity, pools_after_write
from workloads import bits, make_case

pytestmark = pytest.mark.gpu


def _case(hist, ql, seed):
    return make_case("iv", hist_lens=hist, q_lens=ql, write_new=True, causal=False, Hq=8,
                     Hkv=2, D=128, page_size=16, seed=seed, device="cuda")


def _run(case, lo, hi, causal):
    pa.kv_page_write(case.k_pool, case.v_pool, case.k_new, case.v_new, case.cu_new,
                     case.start_pos, case.block_tables)
    out, lse = pa.paged_attn_prefill_varlen(
        case.q, case.k_pool, case.v_pool, case.cu_seqlens_q, case.seq_lens_k,
        case.block_tables, case.scale, causal=causal, max_q_len=case.max_q_len,
        return_lse=True, validate=True,
        key_ranges=(torch.from_numpy(lo).cuda(), torch.from_numpy(hi).cuda()))
    torch.cuda.synchronize()
    return out, lse


def _oracle(case, fn, causal):
    kp, vp = pools_after_write(case)
    return oracle.attention_ref(bits(case.q), kp, vp, case.block_tables.cpu().numpy(),
                                case.seq_lens_k.cpu().numpy(), case.cu_seqlens_q.cpu().numpy(),
                                case.scale, causal, case.page_size, mask_fn=fn)


@pytest.mark.parametrize("prefix", [1, 100, 700])
def test_prefix_lm(require_gpu, prefix):
    """Rows of the prefix see the whole prefix (both ways), later rows are causal:
    row i (position p, no history) sees keys j < max(p + 1, P)."""
    print(f"[interval] prefix-LM P={prefix}", flush=True)
    case = _case([0, 0], [900, 513], 7 + prefix)
    cu = case.cu_seqlens_q.cpu().numpy()
    lens = case.seq_lens
    lo = np.zeros(int(cu[-1]), np.int32)
    hi = np.zeros(int(cu[-1]), np.int32)
    for b in range(2):
        n = int(cu[b + 1] - cu[b])
        pos = lens[b] - n + np.arange(n)
        hi[cu[b]:cu[b + 1]] = np.maximum(pos + 1, min(prefix, lens[b]))
    out, lse = _run(case, lo, hi, causal=False)
    P = [min(prefix, L) for L in lens]
    fn = lambda b, h, q, k: k < np.maximum(q + 1, P[b])
    o_ref, l_ref = _oracle(case, fn, causal=False)
    assert_parity(as_f64(out), o_ref, "prefix-LM")
    assert_lse(as_f64(lse), l_ref, "prefix-LM lse")


@pytest.mark.parametrize("chunk", [64, 200, 1024])
def test_chunked_local_attention(require_gpu, chunk):
    """A row at position p sees the keys of its own chunk of C positions up to itself:
    floor(p / C) C <= j <= p (causal on, key_lo the chunk start)."""
    print(f"[interval] chunked local C={chunk}", flush=True)
    case = _case([300, 0], [700, 1100], 3 + chunk)
    cu = case.cu_seqlens_q.cpu().numpy()
    lens = case.seq_lens
    lo = np.zeros(int(cu[-1]), np.int32)
    hi = np.zeros(int(cu[-1]), np.int32)
    for b in range(2):
        n = int(cu[b + 1] - cu[b])
        pos = lens[b] - n + np.arange(n)
        lo[cu[b]:cu[b + 1]] = (pos // chunk) * chunk
        hi[cu[b]:cu[b + 1]] = lens[b]
    out, lse = _run(case, lo, hi, causal=True)
    n_of = [int(cu[b + 1] - cu[b]) for b in range(2)]
    fn = lambda b, h, q, k: k >= ((lens[b] - n_of[b] + q) // chunk) * chunk
    o_ref, l_ref = _oracle(case, fn, causal=True)
    assert_parity(as_f64(out), o_ref, "chunked local")
    assert_lse(as_f64(lse), l_ref, "chunked local lse")
