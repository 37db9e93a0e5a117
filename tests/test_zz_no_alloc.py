"""paged_attn_decode_noalloc: the decode entry point that allocates nothing (its
split-K partials live in the library's own per-GPU scratch), called through the raw
C ABI and checked against paged_attn_decode with a caller workspace."""

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_flashattention_amd as pa
from paged_kv_flashattention_amd import _lib
from tests.parity import as_f64, assert_lse, assert_parity, oracle_full
from workloads import bits, make_case


def _noalloc(lib, case, out, lse, max_seq_len, S):
    return lib.paged_attn_decode_noalloc(
        out.data_ptr(), lse.data_ptr(), case.q.data_ptr(), case.k_pool.data_ptr(),
        case.v_pool.data_ptr(), case.block_tables.data_ptr(), case.seq_lens_k.data_ptr(),
        case.B, case.max_pages, case.num_pages, case.page_size, case.Hq, case.Hkv, case.D,
        case.scale, max_seq_len, S, torch.cuda.current_stream().cuda_stream)


@pytest.mark.gpu
def test_decode_noalloc_matches_decode_with_a_workspace(require_gpu):
    """Two calls in a row, the second smaller (fewer sequences and splits, so it reads
    only part of what the first left in the scratch): each gives paged_attn_decode's
    bits with a caller workspace and the same split count, and the oracle's result."""
    lib = _lib.load()
    cases = [
        (make_case("na1", seq_lens=[8192, 3000, 17, 5000, 0, 8191, 640, 4096], Hq=28, Hkv=4,
                   D=128, page_size=16, seed=91, device="cuda"), 8192, 16),
        (make_case("na2", seq_lens=[900, 33, 2047], Hq=16, Hkv=2, D=64, page_size=32, seed=92,
                   device="cuda"), 2047, 3),
    ]
    for i, (case, max_len, S) in enumerate(cases):
        print(f"[noalloc] call {i}: B={case.B} Hq={case.Hq} D={case.D} S={S}", flush=True)
        need = pa.decode_workspace_bytes(case.B, case.Hq, case.Hkv, case.D, max_len, S)
        assert 0 < need <= _lib_scratch_bytes()
        ref_o, ref_l = pa.paged_attn_decode(case.q, case.k_pool, case.v_pool,
                                            case.block_tables, case.seq_lens_k, case.scale,
                                            max_seq_len=max_len, num_splits=S,
                                            workspace=torch.empty(need, dtype=torch.uint8,
                                                                  device="cuda"),
                                            return_lse=True)
        out = torch.full_like(ref_o, float("nan"))
        lse = torch.full_like(ref_l, float("nan"))
        st = _noalloc(lib, case, out, lse, max_len, S)
        assert st == 0, lib.pa_last_error()
        assert "decode_partition" in pa.describe_launch()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), bits(ref_o)), i
        assert np.array_equal(lse.cpu().numpy(), ref_l.cpu().numpy()), i
        o_ref, l_ref = oracle_full(case)
        assert_parity(as_f64(out), o_ref, f"noalloc call {i}")
        assert_lse(as_f64(lse), l_ref, f"noalloc lse {i}")


def _lib_scratch_bytes():
    return 32 << 20


def test_decode_noalloc_refuses_partials_beyond_its_scratch():
    """A split count whose partials exceed the 32 MiB scratch is refused on the host
    with PA_ERR_WORKSPACE before the device is touched (no GPU needed)."""
    lib = _lib.load()
    fake = 0x10000
    # 64 x 64 rows x 64 splits x 128 floats = 128 MiB of partials
    st = lib.paged_attn_decode_noalloc(fake, None, fake, fake, fake, fake, fake, 64, 2048,
                                       16384, 64, 64, 8, 128, 0.088, 131072, 64, None)
    assert st == 5
    assert b"scratch" in lib.pa_last_error()
    assert pa.decode_workspace_bytes(64, 64, 8, 128, 131072, 64) > _lib_scratch_bytes()
