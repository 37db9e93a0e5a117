"""GPU kv_page_write: bit-exact against the oracle's scatter."""

import numpy as np
import pytest
import torch

import paged_kv_flashattention_amd as pa
from tests.parity import pools_after_write
from workloads import bits, make_case, make_config

pytestmark = pytest.mark.gpu


def write(case):
    pa.kv_page_write(case.k_pool, case.v_pool, case.k_new, case.v_new, case.cu_new,
                     case.start_pos, case.block_tables, validate=True)
    torch.cuda.synchronize()


@pytest.mark.parametrize("hist,ql,Hkv,D,ps", [
    ([0, 13, 40], [20, 3, 1], 2, 64, 16),
    ([5, 0, 100, 64], [1, 64, 17, 0], 8, 128, 16),
    ([31, 0], [70, 1], 1, 128, 32),
    ([63, 1], [130, 2], 4, 64, 64),
])
def test_kv_write_small(require_gpu, hist, ql, Hkv, D, ps):
    case = make_case("w", hist_lens=hist, q_lens=ql, write_new=True, Hq=Hkv, Hkv=Hkv, D=D,
                     page_size=ps, seed=sum(hist) + D, device="cuda",
                     num_pages=sum(-(-(h + n) // ps) for h, n in zip(hist, ql)) + 3)
    k_ref, v_ref = pools_after_write(case)
    write(case)
    assert np.array_equal(bits(case.k_pool), k_ref)
    assert np.array_equal(bits(case.v_pool), v_ref)


@pytest.mark.parametrize("name", ["mixed_ragged", "causal_prefill"])
def test_kv_write_full_configs(require_gpu, name):
    case = make_config(name, "cuda")
    print(f"[kv_write] {name}: {case.k_new.shape[0]} tokens", flush=True)
    k_ref, v_ref = pools_after_write(case)
    write(case)
    assert np.array_equal(bits(case.k_pool), k_ref)
    assert np.array_equal(bits(case.v_pool), v_ref)


def test_kv_write_no_tokens_is_a_noop(require_gpu):
    case = make_case("w0", hist_lens=[4], q_lens=[0], write_new=True, Hq=2, Hkv=2, D=64,
                     page_size=16, seed=1, device="cuda")
    before = bits(case.k_pool).copy()
    write(case)
    assert np.array_equal(bits(case.k_pool), before)
