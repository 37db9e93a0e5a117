"""GPU parity of document masks (several documents packed into one sequence, each
query row seeing only its own document's keys) against the oracle (reading R6)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_flashattention_amd as pa
from tests.parity import as_f64, assert_lse, assert_parity, oracle_full, pools_after_write
from workloads import bits, document_ranges, make_case

pytestmark = pytest.mark.gpu


def _ranges(case, docs, seed):
    lo, hi = document_ranges(case.seq_lens, case.q_lens, docs, seed)
    return lo, hi, (torch.as_tensor(lo, device="cuda"), torch.as_tensor(hi, device="cuda"))


PREFILL = [
    # hist, q_lens, Hq, Hkv, D, ps, causal, docs, window, alibi, splits
    ([0, 300], [200, 100], 8, 2, 128, 16, True, 3, 0, False, 1),      # 4 waves
    ([0, 0], [1100, 300], 8, 2, 128, 16, True, 5, 0, False, 1),       # 8 waves
    ([500, 0], [600, 513], 8, 4, 128, 32, False, 4, 0, False, 1),     # non-causal: key_hi binds
    ([100, 40], [700, 90], 8, 2, 64, 16, True, 6, 0, False, 1),       # D 64
    ([0, 200], [900, 60], 8, 2, 128, 16, True, 4, 150, False, 1),     # with a window
    ([0, 300], [800, 50], 8, 2, 128, 16, True, 3, 0, True, 1),        # with ALiBi (walk down)
    ([3000, 0], [512, 2500], 8, 2, 128, 16, True, 3, 0, False, 3),    # key parts + merge
    ([2500, 9], [300, 20], 8, 8, 64, 32, False, 2, 0, False, 4),      # key parts, non-causal
]


@pytest.mark.parametrize("hist,ql,Hq,Hkv,D,ps,causal,docs,window,alibi,splits", PREFILL)
def test_prefill_document_masks(require_gpu, hist, ql, Hq, Hkv, D, ps, causal, docs, window,
                                alibi, splits):
    print(f"[documents prefill] hist={hist} q={ql} Hq={Hq} Hkv={Hkv} D={D} causal={causal} "
          f"docs={docs} w={window} alibi={alibi} S={splits}", flush=True)
    case = make_case("pdoc", hist_lens=hist, q_lens=ql, write_new=True, causal=causal, Hq=Hq,
                     Hkv=Hkv, D=D, page_size=ps, seed=sum(hist) + sum(ql) + docs, device="cuda",
                     window=window, num_pages=sum(-(-(h + n) // ps) for h, n in zip(hist, ql)) + 2)
    kp, vp = pools_after_write(case)
    pa.kv_page_write(case.k_pool, case.v_pool, case.k_new, case.v_new, case.cu_new,
                     case.start_pos, case.block_tables, validate=True)
    lo, hi, dev = _ranges(case, docs, sum(ql) + 11)
    slopes = None
    if alibi:
        slopes = torch.tensor([2.0 ** (-(h + 1) / 2) for h in range(Hq)], dtype=torch.float32,
                              device="cuda")
    out, lse = pa.paged_attn_prefill_varlen_splitk(
        case.q, case.k_pool, case.v_pool, case.cu_seqlens_q, case.seq_lens_k, case.block_tables,
        case.scale, causal=causal, max_q_len=case.max_q_len, num_splits=splits, return_lse=True,
        validate=True, window_left=window, alibi_slopes=slopes, key_ranges=dev)
    torch.cuda.synchronize()
    desc = pa.describe_launch()
    if splits > 1:
        assert "prefill_merge" in desc, desc
    o_ref, l_ref = oracle_full(case, kp, vp, alibi=None if slopes is None else slopes.cpu().numpy(),
                               key_ranges=(lo, hi))
    # the masks cut real work: some rows see fewer keys than without documents
    o_nd, _ = oracle_full(case, kp, vp, alibi=None if slopes is None else slopes.cpu().numpy())
    assert np.abs(o_nd - o_ref).max() > 1e-3
    assert_parity(as_f64(out), o_ref, "prefill documents")
    assert_lse(as_f64(lse), l_ref, "prefill documents lse")


def test_prefill_document_masks_fp8_pools(require_gpu):
    """FP8 E4M3 pools with document masks: parity against the oracle's attention over
    the dequantised pools."""
    case = make_case("pdoc8", hist_lens=[100, 0], q_lens=[600, 200], write_new=True,
                     causal=True, Hq=8, Hkv=2, D=128, page_size=16, seed=77, device="cuda")
    kp, vp = pools_after_write(case)
    kf, vf = oracle.bf16_bits_to_f64(kp), oracle.bf16_bits_to_f64(vp)
    # per-pool scales at amax / 448, the generator's poison (NaN, +-3e4) left out
    ks = float(np.float32(np.abs(kf[np.isfinite(kf) & (np.abs(kf) < 1e4)]).max() / 448.0))
    vs = float(np.float32(np.abs(vf[np.isfinite(vf) & (np.abs(vf) < 1e4)]).max() / 448.0))
    kc, vc = oracle.quantize_ref(kp, ks), oracle.quantize_ref(vp, vs)
    k8 = torch.as_tensor(kc, device="cuda")
    v8 = torch.as_tensor(vc, device="cuda")
    lo, hi, dev = _ranges(case, 4, 5)
    out, lse = pa.paged_attn_prefill_varlen_fp8(
        case.q, k8, v8, case.cu_seqlens_q, case.seq_lens_k, case.block_tables, case.scale, ks,
        vs, causal=True, max_q_len=600, return_lse=True, key_ranges=dev)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_ref(
        bits(case.q), oracle.dequantize_pool(kc, ks), oracle.dequantize_pool(vc, vs),
        case.block_tables.cpu().numpy(), case.seq_lens_k.cpu().numpy(),
        case.cu_seqlens_q.cpu().numpy(), case.scale, True, 16, 0, None, (lo, hi))
    assert_parity(as_f64(out), o_ref, "prefill documents fp8")
    assert_lse(as_f64(lse), l_ref, "prefill documents fp8 lse")


@pytest.mark.parametrize("splits", [1, 3, 0])
def test_decode_document_start(require_gpu, splits):
    """Decode rows restricted to their document, which starts anywhere in the
    history (and at the row itself), through the partition kernel and the merge."""
    lens = [3000, 17, 999, 4096, 1, 640]
    case = make_case("ddoc", seq_lens=lens, Hq=28, Hkv=4, D=128, page_size=16, seed=88,
                     device="cuda")
    rng = np.random.default_rng(3)
    lo = np.array([int(rng.integers(0, L)) for L in lens], dtype=np.int32)
    lo[1] = 16                                  # the document is the row itself
    lo[4] = 0
    out, lse = pa.paged_attn_decode(case.q, case.k_pool, case.v_pool, case.block_tables,
                                    case.seq_lens_k, case.scale, max_seq_len=4096,
                                    num_splits=splits, return_lse=True, validate=True,
                                    key_lo=torch.as_tensor(lo, device="cuda"))
    torch.cuda.synchronize()
    hi = np.asarray(lens, dtype=np.int32)
    o_ref, l_ref = oracle_full(case, key_ranges=(lo, hi))
    assert_parity(as_f64(out), o_ref, "decode documents")
    assert_lse(as_f64(lse), l_ref, "decode documents lse")


def test_prefill_documents_are_the_prefill_of_each_document(require_gpu):
    """Causal prefill of three packed documents equals, bit for bit in its choice of
    keys, prefill of each document as a sequence of its own: compared through the
    oracle, and the rows of the first document equal the plain prefill of that
    document alone within the tolerance."""
    case = make_case("pdd", hist_lens=[0], q_lens=[1500], write_new=True, causal=True, Hq=8,
                     Hkv=2, D=128, page_size=16, seed=99, device="cuda")
    kp, vp = pools_after_write(case)
    pa.kv_page_write(case.k_pool, case.v_pool, case.k_new, case.v_new, case.cu_new,
                     case.start_pos, case.block_tables)
    bounds = [0, 700, 1100, 1500]
    lo = np.concatenate([np.full(e - s, s) for s, e in zip(bounds, bounds[1:])]).astype(np.int32)
    hi = np.concatenate([np.full(e - s, e) for s, e in zip(bounds, bounds[1:])]).astype(np.int32)
    out = pa.paged_attn_prefill_varlen(
        case.q, case.k_pool, case.v_pool, case.cu_seqlens_q, case.seq_lens_k, case.block_tables,
        case.scale, causal=True, max_q_len=1500,
        key_ranges=(torch.as_tensor(lo, device="cuda"), torch.as_tensor(hi, device="cuda")))
    # the first document alone: its 700 rows over its own 700 keys
    first = pa.paged_attn_prefill_varlen(
        case.q[:700].contiguous(), case.k_pool, case.v_pool,
        torch.tensor([0, 700], dtype=torch.int32, device="cuda"),
        torch.tensor([700], dtype=torch.int32, device="cuda"), case.block_tables, case.scale,
        causal=True, max_q_len=700)
    torch.cuda.synchronize()
    o_ref, _ = oracle_full(case, kp, vp, key_ranges=(lo, hi))
    assert_parity(as_f64(out), o_ref, "packed documents")
    assert_parity(as_f64(out[:700]), as_f64(first), "first document alone",
                  max_abs=1e-2, mean_abs=1e-3)
