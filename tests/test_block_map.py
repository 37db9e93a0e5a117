"""Prefill with a block map (a mask in block form, 64 query rows x 64 keys per block;
reading R7 of the oracle): the kernel walks only the key tiles a work-group's query
blocks list and masks the rest per query block; the oracle applies the same map as a
predicate on every (row, key)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_flashattention_amd as pa
from tests.parity import as_f64, assert_lse, assert_parity, pools_after_write
from workloads import bits, document_ranges, local_strided_block_map, make_case

pytestmark = pytest.mark.gpu


def random_map(case, density, seed, qb=None, kb=None):
    cu = case.cu_seqlens_q.cpu().numpy()
    lens = case.seq_lens_k.cpu().numpy()
    qb = qb or max(1, -(-int((cu[1:] - cu[:-1]).max()) // 64))
    kb = kb or max(1, -(-int(lens.max()) // 64))
    rng = np.random.default_rng(seed)
    return (rng.random((len(lens), qb, kb)) < density).astype(np.uint8)


def run(case, bm, causal, window=0, alibi=None, key_ranges=None):
    pa.kv_page_write(case.k_pool, case.v_pool, case.k_new, case.v_new, case.cu_new,
                     case.start_pos, case.block_tables)
    out, lse = pa.paged_attn_prefill_varlen(
        case.q, case.k_pool, case.v_pool, case.cu_seqlens_q, case.seq_lens_k,
        case.block_tables, case.scale, causal=causal, max_q_len=case.max_q_len,
        return_lse=True, validate=True, window_left=window, alibi_slopes=alibi,
        key_ranges=None if key_ranges is None else
        (torch.from_numpy(key_ranges[0]).cuda(), torch.from_numpy(key_ranges[1]).cuda()),
        block_map=torch.from_numpy(bm).cuda())
    torch.cuda.synchronize()
    return out, lse


def reference(case, bm, causal, window=0, alibi=None, key_ranges=None, kp=None, vp=None):
    if kp is None:
        kp, vp = pools_after_write(case)
    return oracle.attention_ref(bits(case.q), kp, vp, case.block_tables.cpu().numpy(),
                                case.seq_lens_k.cpu().numpy(), case.cu_seqlens_q.cpu().numpy(),
                                case.scale, causal, case.page_size, window,
                                None if alibi is None else alibi.cpu().numpy(), key_ranges,
                                oracle.block_map_mask(bm))


CASES = [
    # hist, q_lens, Hq, Hkv, D, ps, causal, density
    ([0, 300, 40], [700, 260, 100], 8, 2, 128, 16, True, 0.5),
    ([500, 0], [300, 513], 8, 4, 128, 32, False, 0.3),
    ([100, 40], [600, 90], 8, 2, 64, 64, True, 0.7),
    ([2000, 0, 0], [520, 1100, 64], 16, 4, 128, 16, True, 0.15),
    ([0], [1500], 8, 1, 128, 16, False, 0.9),
]


@pytest.mark.parametrize("hist,ql,Hq,Hkv,D,ps,causal,density", CASES)
def test_block_map_matches_oracle(require_gpu, hist, ql, Hq, Hkv, D, ps, causal, density):
    print(f"[block map] hist={hist} q={ql} Hq={Hq} Hkv={Hkv} D={D} ps={ps} causal={causal} "
          f"density={density}", flush=True)
    case = make_case("bm", hist_lens=hist, q_lens=ql, write_new=True, causal=causal, Hq=Hq,
                     Hkv=Hkv, D=D, page_size=ps, seed=sum(hist) + sum(ql) + D, device="cuda")
    bm = random_map(case, density, sum(ql))
    out, lse = run(case, bm, causal)
    assert "block map" in pa.describe_launch()
    o_ref, l_ref = reference(case, bm, causal)
    assert_parity(as_f64(out), o_ref, "block map")
    assert_lse(as_f64(lse), l_ref, "block map lse")


@pytest.mark.parametrize("what", ["window_documents", "alibi"])
def test_block_map_with_other_masks(require_gpu, what):
    print(f"[block map] with {what}", flush=True)
    case = make_case("bm2", hist_lens=[0, 200], q_lens=[900, 400], write_new=True, causal=True,
                     Hq=8, Hkv=2, D=128, page_size=16, seed=77, device="cuda")
    bm = random_map(case, 0.6, 5)
    if what == "alibi":
        slopes = torch.tensor([2.0 ** (-(h + 1) / 2) for h in range(8)], dtype=torch.float32,
                              device="cuda")
        out, lse = run(case, bm, True, alibi=slopes)
        o_ref, l_ref = reference(case, bm, True, alibi=slopes)
    else:
        kr = document_ranges(case.seq_lens, case.q_lens, 3, 11)
        out, lse = run(case, bm, True, window=300, key_ranges=kr)
        o_ref, l_ref = reference(case, bm, True, window=300, key_ranges=kr)
    assert_parity(as_f64(out), o_ref, f"block map with {what}")
    assert_lse(as_f64(lse), l_ref, f"block map with {what} lse")


def test_block_map_edges(require_gpu):
    """No block listed: every row sees nothing (O = 0, lse = -inf).  Every block
    listed: the mask changes nothing.  A map smaller than the sequences: the keys
    and rows outside it are hidden."""
    case = make_case("bm3", hist_lens=[100, 0], q_lens=[600, 300], write_new=True, causal=True,
                     Hq=8, Hkv=2, D=128, page_size=16, seed=13, device="cuda")
    zeros = np.zeros_like(random_map(case, 0.5, 1))
    out, lse = run(case, zeros, True)
    assert not out.float().abs().sum().item()
    assert bool(torch.all(lse == float("-inf")))
    ones = np.ones_like(zeros)
    out1, lse1 = run(case, ones, True)
    o_ref, l_ref = reference(case, ones, True)
    assert_parity(as_f64(out1), o_ref, "all blocks")
    assert_lse(as_f64(lse1), l_ref, "all blocks lse")
    out0 = pa.paged_attn_prefill_varlen(case.q, case.k_pool, case.v_pool, case.cu_seqlens_q,
                                        case.seq_lens_k, case.block_tables, case.scale,
                                        causal=True, max_q_len=case.max_q_len)
    torch.cuda.synchronize()
    assert_parity(as_f64(out0), o_ref, "no map")
    small = np.ones((2, 2, 3), np.uint8)
    small[0, 1, 0] = 0
    out2, lse2 = run(case, small, True)
    o2, l2 = reference(case, small, True)
    assert_parity(as_f64(out2), o2, "small map")
    assert_lse(as_f64(lse2), l2, "small map lse")


def test_block_map_refusals(require_gpu):
    case = make_case("bm4", hist_lens=[0], q_lens=[300], write_new=True, causal=True, Hq=8,
                     Hkv=2, D=128, page_size=16, seed=1, device="cuda")
    bm = torch.ones((1, 5, 5), dtype=torch.uint8, device="cuda")
    with pytest.raises(TypeError):
        pa.paged_attn_prefill_varlen(case.q, case.k_pool, case.v_pool, case.cu_seqlens_q,
                                     case.seq_lens_k, case.block_tables, case.scale,
                                     max_q_len=300, block_map=bm.int())
    with pytest.raises(ValueError):
        pa.paged_attn_prefill_varlen(case.q, case.k_pool, case.v_pool, case.cu_seqlens_q,
                                     case.seq_lens_k, case.block_tables, case.scale,
                                     max_q_len=300, block_map=bm[0])


def test_block_map_at_full_size_every_work_group(require_gpu):
    """The 4 x 4096 causal prefill (Hq 32, Hkv 8) with a local + strided map: one row
    of every (head, 256-row tile) work-group and whole rows of one head per sequence
    against the oracle, one sampled row at a time."""
    from workloads import make_config
    case = make_config("causal_prefill", device="cuda")
    B = case.seq_lens_k.shape[0]
    m = local_strided_block_map(64, 64)
    bm = np.stack([m] * B)
    pa.kv_page_write(case.k_pool, case.v_pool, case.k_new, case.v_new, case.cu_new,
                     case.start_pos, case.block_tables)
    out, lse = pa.paged_attn_prefill_varlen(case.q, case.k_pool, case.v_pool,
                                            case.cu_seqlens_q, case.seq_lens_k,
                                            case.block_tables, case.scale, causal=True,
                                            max_q_len=case.max_q_len, return_lse=True,
                                            block_map=torch.from_numpy(bm).cuda())
    torch.cuda.synchronize()
    cu = case.cu_seqlens_q.cpu().numpy()
    rng = np.random.default_rng(3)
    rows = []
    for b in range(B):
        for h in range(32):
            for qt in range(16):
                rows.append((int(cu[b]) + qt * 256 + int(rng.integers(0, 256)), h))
        for r in range(0, 4096, 97):
            rows.append((int(cu[b]) + r, 5 + b))
    kp, vp = bits(case.k_pool), bits(case.v_pool)
    ro, rl = oracle.attention_rows_ref(bits(case.q), kp, vp, case.block_tables.cpu().numpy(),
                                       case.seq_lens_k.cpu().numpy(), cu, case.scale, True,
                                       case.page_size, rows,
                                       mask_fn=oracle.block_map_mask(bm))
    got = as_f64(out)[[t for t, _ in rows], [h for _, h in rows]]
    gl = as_f64(lse)[[t for t, _ in rows], [h for _, h in rows]]
    assert_parity(got, ro, "full-size block map")
    assert_lse(gl, rl, "full-size block map lse")


FP8_CASES = [
    # hist, q_lens, Hq, Hkv, D, ps, causal, density, scales, alibi
    ([0, 300, 40], [700, 260, 100], 8, 2, 128, 16, True, 0.5, "pool", False),
    ([500, 0], [300, 513], 8, 4, 128, 32, False, 0.3, "page", False),
    ([100, 40], [600, 90], 8, 2, 64, 64, True, 0.7, "page", False),
    ([0, 200], [900, 400], 8, 2, 128, 16, True, 0.6, "pool", True),
]


@pytest.mark.parametrize("hist,ql,Hq,Hkv,D,ps,causal,density,scales,alibi", FP8_CASES)
def test_block_map_fp8_pools(require_gpu, hist, ql, Hq, Hkv, D, ps, causal, density, scales,
                             alibi):
    """FP8 E4M3 pools (one scale per pool, or per (page, KV head)) with a block map: the
    oracle attends over the same codes dequantised with the same scales."""
    from oracle import fp8 as of
    from workloads import random_e4m3_codes
    print(f"[block map fp8] hist={hist} q={ql} Hq={Hq} Hkv={Hkv} D={D} ps={ps} "
          f"causal={causal} density={density} scales={scales} alibi={alibi}", flush=True)
    case = make_case("bm8", hist_lens=hist, q_lens=ql, write_new=True, causal=causal, Hq=Hq,
                     Hkv=Hkv, D=D, page_size=ps, seed=sum(hist) + sum(ql) + ps, device="cuda")
    shape = tuple(case.k_pool.shape)
    P = shape[0]
    kc = random_e4m3_codes(shape, sum(ql), "cuda")
    vc = random_e4m3_codes(shape, sum(ql) + 1, "cuda")
    rng = np.random.default_rng(sum(hist))
    if scales == "page":
        ks = (2.0 ** rng.uniform(-8, -4, (P, Hkv))).astype(np.float32)
        vs = (2.0 ** rng.uniform(-6, -3, (P, Hkv))).astype(np.float32)
        k_arg, v_arg = torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda()
        kd, vd = of.dequantize_pool(kc.cpu().numpy(), ks), of.dequantize_pool(vc.cpu().numpy(), vs)
    else:
        k_arg, v_arg = 2.0 ** -6, 2.0 ** -4
        kd, vd = of.dequantize_pool(kc.cpu().numpy(), k_arg), of.dequantize_pool(vc.cpu().numpy(), v_arg)
    slopes = None
    if alibi:
        slopes = torch.tensor([2.0 ** (-(h + 1) / 2) for h in range(Hq)], dtype=torch.float32,
                              device="cuda")
    bm = random_map(case, density, sum(ql) + 7)
    out, lse = pa.paged_attn_prefill_varlen_fp8(
        case.q, kc, vc, case.cu_seqlens_q, case.seq_lens_k, case.block_tables, case.scale,
        k_arg, v_arg, causal=causal, max_q_len=case.max_q_len, return_lse=True, validate=True,
        alibi_slopes=slopes, block_map=torch.from_numpy(bm).cuda())
    torch.cuda.synchronize()
    desc = pa.describe_launch()
    assert "block map" in desc and "fp8" in desc.lower(), desc
    o_ref, l_ref = reference(case, bm, causal, alibi=slopes, kp=kd, vp=vd)
    assert_parity(as_f64(out), o_ref, "fp8 block map")
    assert_lse(as_f64(lse), l_ref, "fp8 block map lse")


# ---- decode: the row is query index 0 of its one-row run, so the map is [B, key blocks]

def _decode_oracle(case, bm, kp=None, vp=None, window=0):
    if kp is None:
        kp, vp = bits(case.k_pool), bits(case.v_pool)
    return oracle.attention_ref(bits(case.q), kp, vp, case.block_tables.cpu().numpy(),
                                case.seq_lens_k.cpu().numpy(), case.cu_seqlens_q.cpu().numpy(),
                                case.scale, False, case.page_size, window, None, None,
                                oracle.block_map_mask(bm[:, None, :]))


DECODE_CASES = [
    # lens, Hq, Hkv, D, ps, splits, density
    ([0, 1, 17, 500, 4096, 63, 64, 65], 8, 2, 128, 16, 0, 0.5),
    ([3000, 1000, 129], 28, 4, 128, 32, 3, 0.3),
    ([777, 2048], 16, 8, 64, 64, 1, 0.6),
    ([8192] * 4, 28, 4, 128, 16, 2, 0.1),
]


@pytest.mark.parametrize("lens,Hq,Hkv,D,ps,splits,density", DECODE_CASES)
def test_decode_block_map(require_gpu, lens, Hq, Hkv, D, ps, splits, density):
    print(f"[block map decode] lens={lens} Hq={Hq} Hkv={Hkv} D={D} ps={ps} S={splits} "
          f"density={density}", flush=True)
    case = make_case("bmd", seq_lens=lens, Hq=Hq, Hkv=Hkv, D=D, page_size=ps, seed=sum(lens) + D,
                     device="cuda")
    rng = np.random.default_rng(len(lens))
    bm = (rng.random((len(lens), max(1, -(-max(lens) // 64)))) < density).astype(np.uint8)
    out, lse = pa.paged_attn_decode(case.q, case.k_pool, case.v_pool, case.block_tables,
                                    case.seq_lens_k, case.scale, max_seq_len=max(lens),
                                    num_splits=splits, return_lse=True, validate=True,
                                    block_map=torch.from_numpy(bm).cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = _decode_oracle(case, bm)
    assert_parity(as_f64(out), o_ref, "decode block map")
    assert_lse(as_f64(lse), l_ref, "decode block map lse")


def _sink_window_map(B, L, sink_blocks=1, window_blocks=4):
    """Attention sinks plus a recent window, in block form: the first sink_blocks and
    the last window_blocks 64-key blocks of each sequence."""
    kb = -(-L // 64)
    m = np.zeros((B, kb), np.uint8)
    m[:, :sink_blocks] = 1
    m[:, max(0, kb - window_blocks):] = 1
    return m


def test_decode_block_map_sinks_and_window_full_size(require_gpu):
    """The C2 decode (32 x 8192, Hq 28 / Hkv 4) with sinks + a recent window as a block
    map: every (sequence, head) row against the oracle."""
    from workloads import make_config
    case = make_config("qwen7b_decode", device="cuda")
    bm = _sink_window_map(32, 8192)
    out, lse = pa.paged_attn_decode(case.q, case.k_pool, case.v_pool, case.block_tables,
                                    case.seq_lens_k, case.scale, max_seq_len=8192,
                                    return_lse=True, block_map=torch.from_numpy(bm).cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = _decode_oracle(case, bm)
    assert_parity(as_f64(out), o_ref, "C2 sinks + window")
    assert_lse(as_f64(lse), l_ref, "C2 sinks + window lse")


def test_decode_block_map_fp8_and_window(require_gpu):
    """FP8 pools (scales per page) with a map and a sliding window together."""
    from oracle import fp8 as of
    from workloads import random_e4m3_codes
    case = make_case("bmf", seq_lens=[3000, 700, 1500], Hq=16, Hkv=4, D=128, page_size=16,
                     seed=12, device="cuda")
    shape = tuple(case.k_pool.shape)
    kc, vc = random_e4m3_codes(shape, 1, "cuda"), random_e4m3_codes(shape, 2, "cuda")
    rng = np.random.default_rng(3)
    ks = (2.0 ** rng.uniform(-8, -4, (shape[0], shape[2]))).astype(np.float32)
    vs = (2.0 ** rng.uniform(-6, -3, (shape[0], shape[2]))).astype(np.float32)
    bm = (rng.random((3, 47)) < 0.5).astype(np.uint8)
    out, lse = pa.paged_attn_decode_fp8(case.q, kc, vc, case.block_tables, case.seq_lens_k,
                                        case.scale, torch.from_numpy(ks).cuda(),
                                        torch.from_numpy(vs).cuda(), max_seq_len=3000,
                                        return_lse=True, window_left=1200,
                                        block_map=torch.from_numpy(bm).cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = _decode_oracle(case, bm, of.dequantize_pool(kc.cpu().numpy(), ks),
                                  of.dequantize_pool(vc.cpu().numpy(), vs), window=1200)
    assert_parity(as_f64(out), o_ref, "fp8 decode block map + window")
    assert_lse(as_f64(lse), l_ref, "fp8 decode block map + window lse")
