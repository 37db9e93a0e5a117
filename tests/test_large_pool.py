"""Pools larger than 4 GiB: every kernel addresses pages past the 32-bit byte offset.

Each pool holds 3,000,000 pages of 16 x 1 x 128 bf16 (12.3 GB); the sequences'
pages are a seeded random choice over the whole pool, so most lie beyond 4 GiB.  The
oracle runs on a compact copy of just the pages the sequences use, gathered on
the device, with the block tables renumbered to match.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_flashattention_amd as pa
from tests.parity import as_f64, assert_lse, assert_parity
from workloads import bits

pytestmark = pytest.mark.gpu

P = 3_000_000
PS, HKV, D = 16, 1, 128


def _large_case(lens, q_lens, hist, seed):
    """Pools of P pages on the device, random values only in the pages used."""
    gen = torch.Generator(device="cuda").manual_seed(seed)
    rng = np.random.default_rng(seed)
    k_pool = torch.zeros((P, PS, HKV, D), dtype=torch.bfloat16, device="cuda")
    v_pool = torch.zeros_like(k_pool)
    n_pages = [-(-L // PS) for L in lens]
    pages = rng.choice(P, size=sum(n_pages), replace=False).astype(np.int64)
    assert (pages * PS * HKV * D * 2 >= 1 << 32).mean() > 0.5        # most past 4 GiB
    idx = torch.as_tensor(pages, device="cuda")
    k_pool[idx] = torch.randn((len(pages), PS, HKV, D), generator=gen, device="cuda").to(
        torch.bfloat16)
    v_pool[idx] = torch.randn((len(pages), PS, HKV, D), generator=gen, device="cuda").to(
        torch.bfloat16)
    bt = np.full((len(lens), max(n_pages)), -1, np.int32)
    off = 0
    for b, n in enumerate(n_pages):
        bt[b, :n] = pages[off:off + n]
        off += n
    return k_pool, v_pool, bt, pages


def _compact(pool, bt, pages):
    """The used pages of a device pool as a host array, and the renumbered table."""
    host = bits(pool[torch.as_tensor(pages, device="cuda")])
    remap = {int(p): i for i, p in enumerate(pages)}
    cbt = np.vectorize(lambda x: remap.get(int(x), -1))(bt).astype(np.int32)
    return host, cbt


def test_decode_over_a_pool_larger_than_4gib(require_gpu):
    lens = [3000, 17, 1200, 4096]
    k_pool, v_pool, bt, pages = _large_case(lens, None, None, 41)
    Hq = 8
    q = torch.randn((len(lens), Hq, D), device="cuda").to(torch.bfloat16)
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    bt_t = torch.as_tensor(bt, device="cuda")
    print("[large pool] decode, 12.3 GB pools", flush=True)
    out, lse = pa.paged_attn_decode(q, k_pool, v_pool, bt_t, lens_t, D ** -0.5,
                                    max_seq_len=max(lens), num_splits=3, return_lse=True)
    torch.cuda.synchronize()
    kh, cbt = _compact(k_pool, bt, pages)
    vh, _ = _compact(v_pool, bt, pages)
    o_ref, l_ref = oracle.attention_ref(bits(q), kh, vh, cbt, np.array(lens),
                                        np.arange(len(lens) + 1), D ** -0.5, False, PS)
    assert_parity(as_f64(out), o_ref, "large-pool decode")
    assert_lse(as_f64(lse), l_ref, "large-pool decode lse")


def test_write_and_prefill_over_a_pool_larger_than_4gib(require_gpu):
    hist, q_lens = [2000, 0, 700], [300, 513, 64]
    lens = [h + n for h, n in zip(hist, q_lens)]
    k_pool, v_pool, bt, pages = _large_case(lens, q_lens, hist, 42)
    Hq, T = 4, sum(q_lens)
    q = torch.randn((T, Hq, D), device="cuda").to(torch.bfloat16)
    k_new = torch.randn((T, HKV, D), device="cuda").to(torch.bfloat16)
    v_new = torch.randn((T, HKV, D), device="cuda").to(torch.bfloat16)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]), dtype=torch.int32,
                      device="cuda")
    sp = torch.tensor(hist, dtype=torch.int32, device="cuda")
    bt_t = torch.as_tensor(bt, device="cuda")
    kh0, cbt = _compact(k_pool, bt, pages)
    vh0, _ = _compact(v_pool, bt, pages)
    print("[large pool] write + prefill, 12.3 GB pools", flush=True)
    pa.kv_page_write(k_pool, v_pool, k_new, v_new, cu, sp, bt_t)
    out, lse = pa.paged_attn_prefill_varlen(q, k_pool, v_pool, cu,
                                            torch.tensor(lens, dtype=torch.int32, device="cuda"),
                                            bt_t, D ** -0.5, causal=True, max_q_len=513,
                                            return_lse=True)
    torch.cuda.synchronize()
    # the write, bit for bit, on the compact copy
    kw, vw = oracle.kv_write_ref(kh0, vh0, bits(k_new), bits(v_new), cu.cpu().numpy(),
                                 np.array(hist), cbt, PS)
    kh, _ = _compact(k_pool, bt, pages)
    vh, _ = _compact(v_pool, bt, pages)
    assert np.array_equal(kh, kw) and np.array_equal(vh, vw)
    o_ref, l_ref = oracle.attention_ref(bits(q), kw, vw, cbt, np.array(lens),
                                        cu.cpu().numpy(), D ** -0.5, True, PS)
    assert_parity(as_f64(out), o_ref, "large-pool prefill")
    assert_lse(as_f64(lse), l_ref, "large-pool prefill lse")
