"""Grouped decode partitions: when a caller's split count asks for several times more
one-wave work-groups than the decode streams best with, a one-wave work-group walks
several consecutive partitions of one (KV head, sequence), each with the partition
kernel's own walk.  The partials, and so the outputs, must be the bits of the same
batch computed one partition per one-wave work-group: checked against sub-batches
small enough to launch that way, and against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_flashattention_amd as pa
from oracle import fp8 as of
from tests.parity import as_f64, assert_lse, assert_parity, oracle_full
from workloads import bits, make_case

pytestmark = pytest.mark.gpu


def _target(fp8):
    # one-wave work-groups the decode streams best with on MI355X (two / four per CU)
    return 1024 if fp8 else 512


def _group(B, Hkv, S, fp8):
    g = B * Hkv * S // _target(fp8)
    return 1 if g < 2 else min(g, S)


def _sub_batch(Hkv, S, fp8):
    """Sequences per sub-batch whose launch is one one-wave work-group per partition."""
    n = -(-_target(fp8) // (Hkv * S))
    assert n * Hkv * S < 2 * _target(fp8)
    return n


def _slice(case, b0, b1):
    return (case.q[b0:b1].contiguous(), case.block_tables[b0:b1].contiguous(),
            case.seq_lens_k[b0:b1].contiguous())


def _decode(case, q, bt, sl, S, fp8=None, block_map=None, **extra):
    kw = dict(max_seq_len=case.max_seq_len, num_splits=S, return_lse=True, validate=True,
              block_map=block_map, **extra)
    if fp8 is None:
        out, lse = pa.paged_attn_decode(q, case.k_pool, case.v_pool, bt, sl, case.scale, **kw)
    else:
        kc, vc, ks, vs = fp8
        out, lse = pa.paged_attn_decode_fp8(q, kc, vc, bt, sl, case.scale, ks, vs, **kw)
    torch.cuda.synchronize()
    return out, lse, pa.describe_launch()


def _check_against_sub_batches(case, S, fp8=None, block_map=None, key_lo=None, **extra):
    """The grouped launch over the whole batch, then each sub-batch launched one
    partition per one-wave work-group: equal bits, row by row."""
    B, Hkv = case.q.shape[0], case.k_pool.shape[2]
    g = _group(B, Hkv, S, fp8 is not None)
    assert g >= 2
    out, lse, desc = _decode(case, case.q, case.block_tables, case.seq_lens_k, S, fp8, block_map,
                             key_lo=key_lo, **extra)
    assert "decode_group" in desc and f"partitions per work-group={g}" in desc, desc
    n = _sub_batch(Hkv, S, fp8 is not None)
    assert B % n == 0
    for b0 in range(0, B, n):
        bm = None if block_map is None else block_map[b0:b0 + n].contiguous()
        lo = None if key_lo is None else key_lo[b0:b0 + n].contiguous()
        o, l, d = _decode(case, *_slice(case, b0, b0 + n), S, fp8, bm, key_lo=lo, **extra)
        assert "decode_partition" in d and "W=1" in d, d
        assert torch.equal(out[b0:b0 + n].view(torch.int16), o.view(torch.int16)), (b0, desc)
        assert torch.equal(lse[b0:b0 + n], l), (b0, desc)
    return out, lse


def _lens(B, hi, mult, zero_every=5):
    return [0 if i % zero_every == 0 else (mult * i) % hi + 1 for i in range(B)]


BF16 = [
    # B, Hq, Hkv, D, ps, splits, max length
    (16, 16, 8, 128, 16, 8, 3001),      # 1,024 partitions: 2 per work-group
    (16, 64, 8, 64, 64, 16, 4097),      # 2,048: 4, GQA 8, page 64, D 64
    (30, 8, 8, 128, 32, 7, 2000),       # 1,680: 3 (the last group of each row holds 1)
    (8, 16, 8, 128, 16, 64, 9000),      # 4,096: 8 (most partitions of short rows empty)
]


@pytest.mark.parametrize("B,Hq,Hkv,D,ps,splits,hi", BF16)
def test_grouped_partitions_bf16(require_gpu, B, Hq, Hkv, D, ps, splits, hi):
    lens = _lens(B, hi, 977)
    print(f"[decode group] bf16 B={B} Hq={Hq} Hkv={Hkv} D={D} ps={ps} S={splits}", flush=True)
    case = make_case("grp", seq_lens=lens, Hq=Hq, Hkv=Hkv, D=D, page_size=ps,
                     seed=sum(lens) + D + splits, device="cuda")
    out, lse = _check_against_sub_batches(case, splits)
    o_ref, l_ref = oracle_full(case)
    assert_parity(as_f64(out), o_ref, "grouped decode")
    assert_lse(as_f64(lse), l_ref, "grouped decode lse")
    for b, L in enumerate(lens):
        if L == 0:
            assert (as_f64(out[b]) == 0).all() and np.isneginf(as_f64(lse[b])).all()


def test_grouped_partials_equal_one_partition_per_work_group(require_gpu):
    """The per-partition partials (output and lse, empty partitions included) of a
    grouped launch are the bits of the ungrouped sub-batches' partials."""
    B, Hq, Hkv, D, ps, S = 16, 16, 8, 128, 16, 8
    lens = _lens(B, 2500, 613)
    case = make_case("grpp", seq_lens=lens, Hq=Hq, Hkv=Hkv, D=D, page_size=ps, seed=77,
                     device="cuda")
    print("[decode group] partials", flush=True)
    po, pl = pa.paged_attn_decode_partials(case.q, case.k_pool, case.v_pool, case.block_tables,
                                           case.seq_lens_k, case.scale, S,
                                           max_seq_len=case.max_seq_len)
    torch.cuda.synchronize()
    assert "partitions per work-group=2" in pa.describe_launch()
    n = _sub_batch(Hkv, S, False)
    for b0 in range(0, B, n):
        q, bt, sl = _slice(case, b0, b0 + n)
        o, l = pa.paged_attn_decode_partials(q, case.k_pool, case.v_pool, bt, sl, case.scale, S,
                                             max_seq_len=case.max_seq_len)
        torch.cuda.synchronize()
        assert "decode_partition" in pa.describe_launch()
        rows = slice(b0 * Hq, (b0 + n) * Hq)
        assert torch.equal(po[rows], o) and torch.equal(pl[rows], l), b0
    # each partition against the oracle's partials over the same boundaries (a
    # partition with no key: O = 0, lse = -inf), for every third sequence
    part_len = -(-(-(-case.max_seq_len // 32)) // S) * 32
    kp, vp = bits(case.k_pool), bits(case.v_pool)
    bt = case.block_tables.cpu().numpy()
    q = oracle.bf16_bits_to_f64(bits(case.q))
    got_o, got_l = po.cpu().numpy(), pl.cpu().numpy()
    G = Hq // Hkv
    for b in range(0, B, 3):
        L = lens[b]
        k = oracle.gather_sequence_kv(kp, bt[b], L, ps)
        v = oracle.gather_sequence_kv(vp, bt[b], L, ps)
        bounds = [min(c * part_len, L) for c in range(S)] + [L]
        for h in range(Hq):
            oc, lc = oracle.split_partials_ref(q[b, h], k[:, h // G], v[:, h // G], case.scale,
                                               L, bounds)
            r = b * Hq + h
            assert_parity(got_o[r], oc, f"partials b={b} h={h}", max_abs=2e-3, mean_abs=2e-4)
            assert_lse(got_l[r], lc, f"partial lse b={b} h={h}")


FP8 = [
    # B, Hq, Hkv, D, ps, splits, max length, scales per page
    (16, 32, 8, 128, 16, 32, 6000, False),   # 4,096 partitions: 4 per work-group
    (16, 16, 8, 64, 32, 16, 3000, True),     # 2,048: 2, D 64, scales per (page, KV head)
]


@pytest.mark.parametrize("B,Hq,Hkv,D,ps,splits,hi,per_page", FP8)
def test_grouped_partitions_fp8(require_gpu, B, Hq, Hkv, D, ps, splits, hi, per_page):
    lens = _lens(B, hi, 1409)
    print(f"[decode group] fp8 B={B} Hq={Hq} Hkv={Hkv} D={D} ps={ps} S={splits} "
          f"per_page={per_page}", flush=True)
    case = make_case("grp8", seq_lens=lens, Hq=Hq, Hkv=Hkv, D=D, page_size=ps,
                     seed=sum(lens) + D + 8, device="cuda")
    kb, vb = bits(case.k_pool), bits(case.v_pool)
    if per_page:
        P = case.k_pool.shape[0]
        rng = np.random.default_rng(sum(lens))
        ks = (2.0 ** rng.uniform(-7, -5, (P, Hkv))).astype(np.float32)
        vs = (2.0 ** rng.uniform(-7, -5, (P, Hkv))).astype(np.float32)
        kc, vc = of.quantize_ref(kb, of.page_scales(ks)), of.quantize_ref(vb, of.page_scales(vs))
        kd, vd = of.dequantize_pool(kc, ks), of.dequantize_pool(vc, vs)
        k_s, v_s = torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda()
    else:
        x = np.abs(oracle.bf16_bits_to_f64(kb))
        ks = float(np.float32(x[np.isfinite(x) & (x < 1e4)].max() / 448.0))
        x = np.abs(oracle.bf16_bits_to_f64(vb))
        vs = float(np.float32(x[np.isfinite(x) & (x < 1e4)].max() / 448.0))
        kc, vc = of.quantize_ref(kb, ks), of.quantize_ref(vb, vs)
        kd, vd = of.dequantize_pool(kc, ks), of.dequantize_pool(vc, vs)
        k_s, v_s = ks, vs
    fp8 = (torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda(), k_s, v_s)
    out, lse = _check_against_sub_batches(case, splits, fp8)
    o_ref, l_ref = oracle_full(case, kd, vd)
    assert_parity(as_f64(out), o_ref, "grouped fp8 decode")
    assert_lse(as_f64(lse), l_ref, "grouped fp8 decode lse")


def test_grouped_partitions_block_map(require_gpu):
    """A block map with grouped partitions: the walk visits only listed tiles in
    each partition of the group."""
    B, Hq, Hkv, D, ps, S = 16, 16, 8, 128, 16, 16
    lens = _lens(B, 5000, 1231)
    case = make_case("grpm", seq_lens=lens, Hq=Hq, Hkv=Hkv, D=D, page_size=ps, seed=91,
                     device="cuda")
    rng = np.random.default_rng(92)
    bm = (rng.random((B, -(-max(lens) // 64))) < 0.3).astype(np.uint8)
    print("[decode group] block map", flush=True)
    out, lse = _check_against_sub_batches(case, S, block_map=torch.from_numpy(bm).cuda())
    o_ref, l_ref = oracle.attention_ref(bits(case.q), bits(case.k_pool), bits(case.v_pool),
                                        case.block_tables.cpu().numpy(),
                                        case.seq_lens_k.cpu().numpy(),
                                        case.cu_seqlens_q.cpu().numpy(), case.scale, False,
                                        case.page_size, 0, None, None,
                                        oracle.block_map_mask(bm[:, None, :]))
    assert_parity(as_f64(out), o_ref, "grouped decode block map")
    assert_lse(as_f64(lse), l_ref, "grouped decode block map lse")


def test_grouped_partitions_window_alibi_documents(require_gpu):
    """Grouped partitions with a sliding window, ALiBi slopes and document starts, which
    move where each row's walk begins (partitions sized for the window)."""
    B, Hq, Hkv, D, ps, S, w = 16, 16, 8, 128, 16, 16, 3000
    lens = _lens(B, 9000, 1571)
    case = make_case("grpw", seq_lens=lens, Hq=Hq, Hkv=Hkv, D=D, page_size=ps, seed=93,
                     device="cuda", window=w)
    rng = np.random.default_rng(94)
    lo = np.array([int(rng.integers(0, L)) if L else 0 for L in lens], dtype=np.int32)
    slopes = torch.from_numpy((2.0 ** -rng.uniform(1, 8, Hq)).astype(np.float32)).cuda()
    print("[decode group] window + alibi + documents", flush=True)
    out, lse = _check_against_sub_batches(case, S, key_lo=torch.from_numpy(lo).cuda(),
                                          window_left=w, alibi_slopes=slopes)
    o_ref, l_ref = oracle_full(case, alibi=slopes.cpu().numpy(),
                               key_ranges=(lo, np.asarray(lens, dtype=np.int32)))
    assert_parity(as_f64(out), o_ref, "grouped decode window alibi documents")
    assert_lse(as_f64(lse), l_ref, "grouped decode window alibi documents lse")
