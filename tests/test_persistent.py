"""Persistent prefill work-groups (pa_prefill_opts.persistent): each work-group takes
the plain grid's items in turn, prefetching the next item's Q rows and first K/V tile.
The arithmetic per item is the plain kernel's, so the results are the same bits; the
oracle checks them too."""

import pytest
import torch

import paged_kv_flashattention_amd as pa
from tests.parity import as_f64, assert_lse, assert_parity, oracle_full
from workloads import make_case

pytestmark = pytest.mark.gpu

CASES = [
    # hist, q_lens, Hq, Hkv, D, causal, splits
    ([0, 0, 0], [1024, 700, 513], 8, 2, 128, True, 1),       # more items than one round
    ([300, 0, 5000], [512, 1, 600], 16, 4, 128, True, 1),    # an item without tiles' rows
    ([2000, 100], [600, 512], 8, 2, 128, False, 1),          # non-causal
    ([4000, 0], [520, 900], 8, 1, 128, True, 3),             # key parts, merged
    ([0, 700], [1100, 530], 8, 2, 64, True, 1),              # D 64
    ([0], [4096], 32, 8, 128, True, 1),                      # many heavy items
]


@pytest.mark.parametrize("hist,ql,Hq,Hkv,D,causal,splits", CASES)
def test_persistent_matches_plain_grid_bits(require_gpu, hist, ql, Hq, Hkv, D, causal, splits):
    print(f"[persistent] hist={hist} q={ql} Hq={Hq} Hkv={Hkv} D={D} causal={causal} "
          f"S={splits}", flush=True)
    case = make_case("per", hist_lens=hist, q_lens=ql, write_new=True, causal=causal, Hq=Hq,
                     Hkv=Hkv, D=D, page_size=16, seed=sum(hist) + sum(ql) + D, device="cuda")
    pa.kv_page_write(case.k_pool, case.v_pool, case.k_new, case.v_new, case.cu_new,
                     case.start_pos, case.block_tables)
    if splits > 1:
        kw = dict(num_splits=splits)
        fn = pa.paged_attn_prefill_varlen_splitk
    else:
        kw = {}
        fn = pa.paged_attn_prefill_varlen
    o0, l0 = fn(case.q, case.k_pool, case.v_pool, case.cu_seqlens_q, case.seq_lens_k,
                case.block_tables, case.scale, causal=causal, max_q_len=case.max_q_len,
                return_lse=True, **kw)
    torch.cuda.synchronize()
    plain = pa.describe_launch()
    o1, l1 = fn(case.q, case.k_pool, case.v_pool, case.cu_seqlens_q, case.seq_lens_k,
                case.block_tables, case.scale, causal=causal, max_q_len=case.max_q_len,
                return_lse=True, persistent=True, **kw)
    torch.cuda.synchronize()
    desc = pa.describe_launch()
    if case.max_q_len >= 512:
        assert "persistent" in desc, desc
    assert "persistent" not in plain
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l0.view(torch.int32), l1.view(torch.int32))
    o_ref, l_ref = oracle_full(case)
    assert_parity(as_f64(o1), o_ref, "persistent prefill")
    assert_lse(as_f64(l1), l_ref, "persistent prefill lse")


def test_persistent_is_ignored_where_it_does_not_apply(require_gpu):
    """Query runs below 512 rows take 128-row tiles, a window the general variant:
    the option is a hint, and the plain grid runs."""
    case = make_case("per2", hist_lens=[100], q_lens=[300], write_new=True, causal=True, Hq=8,
                     Hkv=2, D=128, page_size=16, seed=3, device="cuda", window=64)
    pa.kv_page_write(case.k_pool, case.v_pool, case.k_new, case.v_new, case.cu_new,
                     case.start_pos, case.block_tables)
    o = pa.paged_attn_prefill_varlen(case.q, case.k_pool, case.v_pool, case.cu_seqlens_q,
                                     case.seq_lens_k, case.block_tables, case.scale,
                                     causal=True, max_q_len=300, window_left=64,
                                     persistent=True)
    torch.cuda.synchronize()
    assert "persistent" not in pa.describe_launch()
    o_ref, _ = oracle_full(case)
    assert_parity(as_f64(o), o_ref, "window with the persistent hint")
