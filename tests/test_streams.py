"""Launch streams other than the current one, and prepared() replays: buffers the
binding allocates for a call (outputs, workspaces) must stay the call's while the
launch stream's kernels use them."""

import numpy as np
import pytest
import torch

import paged_kv_flashattention_amd as pa
from tests.parity import as_f64, assert_parity, oracle_full
from workloads import bits, make_case

pytestmark = pytest.mark.gpu


def _churn():
    """Allocate and fill blocks on the current stream: with a buffer of a call on
    another stream freed too early, one of these would land on it."""
    junk = [torch.full((n,), 0x7F, dtype=torch.uint8, device="cuda")
            for n in (1 << 16, 1 << 20, 1 << 22, 1 << 24)]
    junk += [torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
             for n in (1 << 14, 1 << 18, 1 << 21)]
    return junk


def test_decode_and_prefill_on_a_non_current_stream(require_gpu):
    dec = make_case("sd", seq_lens=[3000, 17, 999, 4096], Hq=28, Hkv=4, D=128, page_size=16,
                    seed=81, device="cuda")
    pf = make_case("sp", seq_lens=[4000, 600], q_lens=[64, 600], Hq=8, Hkv=2, D=128,
                   page_size=16, seed=82, causal=True, device="cuda")
    d_args = (dec.q, dec.k_pool, dec.v_pool, dec.block_tables, dec.seq_lens_k, dec.scale)
    p_args = (pf.q, pf.k_pool, pf.v_pool, pf.cu_seqlens_q, pf.seq_lens_k, pf.block_tables,
              pf.scale)
    ref_d = bits(pa.paged_attn_decode(*d_args, max_seq_len=4096, num_splits=5))
    ref_p = bits(pa.paged_attn_prefill_varlen_splitk(*p_args, max_q_len=600, num_splits=4))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        # launched on `side` with every buffer allocated by the binding, while the
        # current stream goes on allocating
        out_d = pa.paged_attn_decode(*d_args, max_seq_len=4096, num_splits=5, stream=side)
        out_p = pa.paged_attn_prefill_varlen_splitk(*p_args, max_q_len=600, num_splits=4,
                                                    stream=side.cuda_stream)
        junk = _churn()
        side.synchronize()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out_d), ref_d), rep
        assert np.array_equal(bits(out_p), ref_p), rep
        del junk, out_d, out_p
    assert_parity(as_f64(torch.as_tensor(ref_d.view(np.int16)).view(torch.bfloat16)),
                  oracle_full(dec)[0], "decode on a side stream")


def test_prepared_replay_keeps_its_own_buffers(require_gpu):
    """A prepared call whose output and split-K workspace the binding allocated replays
    into those same buffers, which no other allocation receives in the meantime: the
    replays give the first call's bits, and blocks allocated between replays keep
    what was written into them."""
    case = make_case("pr", seq_lens=[5000, 300, 8192], Hq=28, Hkv=4, D=128, page_size=16,
                     seed=83, device="cuda")
    holder = {}

    def call():
        holder["out"] = pa.paged_attn_decode(case.q, case.k_pool, case.v_pool,
                                             case.block_tables, case.seq_lens_k, case.scale,
                                             max_seq_len=8192, num_splits=4)
    run = pa.prepared(call)
    torch.cuda.synchronize()
    out = holder.pop("out")
    ref = bits(out).copy()
    assert_parity(as_f64(out), oracle_full(case)[0], "prepared decode")
    torch.cuda.empty_cache()
    for rep in range(3):
        out.zero_()
        junk = _churn()
        run()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), ref), rep
        for j in junk:
            if j.dtype == torch.uint8:
                assert bool((j == 0x7F).all()), rep
            else:
                assert bool(torch.isnan(j).all()), rep
        del junk
