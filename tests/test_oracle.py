"""Pins for the float64 oracle: it must agree with things other than itself.

* brute force: pure-Python loops with math.exp / math.fsum and a page walk
  written here, on tiny random inputs;
* a library routine: torch's float64 CPU scaled_dot_product_attention with
  an explicit mask, and scipy's logsumexp for the lse;
* closed forms: one key, constant V, Q = 0, a dominant key, an empty row;
* invariants: softmax rows sum to one, page permutation, page size, GQA as
  repeated MHA, tiled == untiled for any tile, split + merge == unsplit for
  any partition, last causal row == decode, chunked prefill == one shot;
* the traffic figures the pages print (tests/golden/traffic_figures.json);
* planted mistakes: each plausible oracle bug must fail one of the pins.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st
from scipy.special import logsumexp

import oracle
from oracle import attention as oa
from workloads import bits, document_ranges, make_case, units

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# brute force, written independently of the oracle
# ----------------------------------------------------------------------------

def _bf16(x):
    x = np.asarray(x, dtype=np.uint16)
    return [float(np.frombuffer(np.uint32(int(v) << 16).tobytes(), dtype=np.float32)[0])
            for v in x.ravel()]


def brute_attention(case, window=None, alibi=None, key_ranges=None, pred=None):
    """Loops over sequences, rows, heads and keys; math.exp and math.fsum only.
    With a sliding window w > 0 the row at position p takes keys j > p - w only;
    with ALiBi slopes the score of key j gets slope_h * (j - p) added; with
    document ranges (key_lo, key_hi) per row, row t takes keys key_lo[t] <= j <
    key_hi[t] only; with a predicate, row i of sequence b (i counted within its
    query run) and head h take key j only if pred(b, h, i, j) is true."""
    w = case.window if window is None else window
    q = bits(case.q)
    kp = bits(case.k_pool)
    vp = bits(case.v_pool)
    bt = case.block_tables.numpy()
    lens = case.seq_lens_k.numpy()
    cu = case.cu_seqlens_q.numpy()
    T, Hq, D = q.shape
    Hkv, ps = kp.shape[2], kp.shape[1]
    grp = Hq // Hkv
    out = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -np.inf)
    for b in range(len(lens)):
        L = int(lens[b])
        n = int(cu[b + 1] - cu[b])
        for i in range(n):
            t = int(cu[b]) + i
            limit = L if not case.causal else L - n + i + 1
            pos = L - n + i
            start = pos - w + 1 if w > 0 else 0
            for h in range(Hq):
                kvh = h // grp
                qv = _bf16(q[t, h])
                scores, vrows = [], []
                for j in range(max(0, min(limit, L))):
                    if j < start:
                        continue
                    if key_ranges is not None and not (key_ranges[0][t] <= j < key_ranges[1][t]):
                        continue
                    if pred is not None and not bool(pred(b, h, i, j)):
                        continue
                    page, slot = int(bt[b][j // ps]), j % ps
                    kv = _bf16(kp[page, slot, kvh])
                    bias = 0.0 if alibi is None else float(alibi[h]) * (j - pos)
                    scores.append(case.scale * math.fsum(a * c for a, c in zip(qv, kv)) + bias)
                    vrows.append(_bf16(vp[page, slot, kvh]))
                if not scores:
                    continue
                m = max(scores)
                e = [math.exp(s - m) for s in scores]
                den = math.fsum(e)
                for d in range(D):
                    out[t, h, d] = math.fsum(w * vr[d] for w, vr in zip(e, vrows)) / den
                lse[t, h] = m + math.log(den)
    return out, lse


def run_oracle(case, window=None, alibi=None, key_ranges=None):
    return oracle.attention_ref(bits(case.q), bits(case.k_pool), bits(case.v_pool),
                                case.block_tables.numpy(), case.seq_lens_k.numpy(),
                                case.cu_seqlens_q.numpy(), case.scale, case.causal,
                                case.page_size, case.window if window is None else window,
                                alibi, key_ranges)


def assert_close(a, b, tol=1e-12):
    a, b = np.asarray(a), np.asarray(b)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    assert np.array_equal(a[~fin], b[~fin])
    if fin.any():
        err = np.abs(a[fin] - b[fin]) / (1.0 + np.abs(b[fin]))
        assert err.max() <= tol, err.max()


small_shapes = st.fixed_dictionaries(dict(
    B=st.integers(1, 3),
    D=st.sampled_from([4, 8]),
    Hkv=st.integers(1, 2),
    G=st.sampled_from([1, 2, 3, 7]),
    ps=st.sampled_from([1, 3, 16]),
    causal=st.booleans(),
    seed=st.integers(0, 10_000),
    lens=st.lists(st.integers(0, 40), min_size=3, max_size=3),
    qlens=st.lists(st.integers(1, 5), min_size=3, max_size=3),
    window=st.sampled_from([0, 0, 1, 2, 5, 17]),
    docs=st.sampled_from([0, 0, 1, 3]),
))


def _small_case(p):
    B = p["B"]
    lens = p["lens"][:B]
    ql = [min(n, max(L, 1)) for n, L in zip(p["qlens"][:B], lens)]
    spare = 3
    return make_case("hyp", seq_lens=lens, q_lens=ql, Hq=p["Hkv"] * p["G"], Hkv=p["Hkv"],
                     D=p["D"], page_size=p["ps"], seed=p["seed"], causal=p["causal"],
                     num_pages=sum(-(-L // p["ps"]) for L in lens) + spare,
                     window=p["window"])


@settings(max_examples=40, deadline=None)
@given(small_shapes)
def test_oracle_matches_brute_force(p):
    case = _small_case(p)
    kr = document_ranges(case.seq_lens, case.q_lens, p["docs"], p["seed"]) if p["docs"] else None
    o, lse = run_oracle(case, key_ranges=kr)
    ob, lseb = brute_attention(case, key_ranges=kr)
    assert_close(o, ob)
    assert_close(lse, lseb)


def test_brute_force_covers_poison_and_tails():
    # partially filled last pages, an empty sequence, spare NaN pages, GQA 7
    case = make_case("t", seq_lens=[0, 5, 33], q_lens=[1, 3, 4], Hq=7, Hkv=1, D=8,
                     page_size=16, num_pages=8, seed=3, causal=True)
    o, lse = run_oracle(case)
    assert np.isfinite(o).all()
    ob, lseb = brute_attention(case)
    assert_close(o, ob)
    assert_close(lse, lseb)
    assert (lse[0] == -np.inf).all() and (o[0] == 0).all()


# ----------------------------------------------------------------------------
# library routines
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("L,n", [(1, 1), (17, 1), (64, 64), (100, 37)])
def test_attend_rows_matches_torch_sdpa_float64(L, n, causal):
    rng = np.random.default_rng(L * 31 + n)
    D = 16
    q = rng.standard_normal((n, D))
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    vis = oa._visible_counts(L, n, causal)
    o, lse = oracle.attend_rows(q, k, v, 0.3, vis)
    mask = torch.arange(L)[None, :] < torch.as_tensor(vis)[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(q)[None], torch.as_tensor(k)[None], torch.as_tensor(v)[None],
        attn_mask=mask[None], scale=0.3)[0].numpy()
    assert np.abs(o - ref).max() < 1e-12
    s = 0.3 * q @ k.T
    s[~mask.numpy()] = -np.inf
    assert np.abs(lse - logsumexp(s, axis=1)).max() < 1e-12


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------

def test_single_key_returns_its_value_row():
    rng = np.random.default_rng(1)
    q, k, v = rng.standard_normal((3, 8)), rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    o, lse = oracle.attend_rows(q, k, v, 0.5, [1, 1, 1])
    assert np.array_equal(o, np.repeat(v, 3, axis=0))
    assert np.allclose(lse, 0.5 * q @ k[0], rtol=0, atol=1e-14)


def test_constant_values_return_that_constant():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((4, 8)), rng.standard_normal((50, 8))
    v = np.tile(rng.standard_normal(8), (50, 1))
    o, _ = oracle.attend_rows(q, k, v, 1.0, [50, 10, 1, 33])
    assert np.abs(o - v[0]).max() < 1e-13


def test_zero_query_returns_mean_of_visible_values():
    rng = np.random.default_rng(3)
    k, v = rng.standard_normal((40, 8)), rng.standard_normal((40, 8))
    o, lse = oracle.attend_rows(np.zeros((3, 8)), k, v, 1.0, [40, 7, 1])
    for i, n in enumerate([40, 7, 1]):
        assert np.abs(o[i] - v[:n].mean(axis=0)).max() < 1e-13
        assert abs(lse[i] - math.log(n)) < 1e-13


def test_dominant_key_returns_its_value_row():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((64, 8)) * 0.01
    v = rng.standard_normal((64, 8))
    q = np.zeros((1, 8))
    q[0, 0] = 1.0
    k[17, 0] = 200.0                               # score gap >= 110
    o, _ = oracle.attend_rows(q, k, v, 1.0, [64])
    assert np.abs(o[0] - v[17]).max() < 1e-40


def test_fully_masked_row_is_zero_with_minus_inf_lse():
    rng = np.random.default_rng(5)
    k, v = rng.standard_normal((5, 4)), rng.standard_normal((5, 4))
    o, lse = oracle.attend_rows(rng.standard_normal((2, 4)), k, v, 1.0, [0, 3])
    assert (o[0] == 0).all() and lse[0] == -np.inf
    assert np.isfinite(o[1]).all()
    o, lse = oracle.attend_rows(np.ones((1, 4)), np.zeros((0, 4)), np.zeros((0, 4)), 1.0, [0])
    assert (o == 0).all() and lse[0] == -np.inf


def test_extreme_logits_stay_finite_and_match_brute_force():
    case = make_case("x", seq_lens=[37, 100], Hq=4, Hkv=2, D=8, page_size=16, seed=7)
    case.q = (case.q.float() * 30).to(torch.bfloat16)
    o, lse = run_oracle(case)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    ob, lseb = brute_attention(case)
    assert_close(o, ob, 1e-11)
    assert_close(lse, lseb, 1e-11)


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------

def test_softmax_rows_sum_to_one_and_masked_keys_are_zero():
    rng = np.random.default_rng(6)
    q, k = rng.standard_normal((5, 8)), rng.standard_normal((30, 8))
    vis = [30, 1, 15, 0, 29]
    p = oracle.softmax_probs_ref(q, k, 0.7, vis)
    for i, n in enumerate(vis):
        assert (p[i, n:] == 0).all()
        if n:
            assert abs(p[i].sum() - 1.0) < 1e-12
        else:
            assert (p[i] == 0).all()


def _brute_probs(q, k, scale, vis):
    """Softmax probabilities by pure-Python loops: scaled dot products summed with
    math.fsum, natural exponentials of the shifted scores, division by their sum."""
    n, L = len(q), len(k)
    p = [[0.0] * L for _ in range(n)]
    for i in range(n):
        s = [scale * math.fsum(float(a) * float(b) for a, b in zip(q[i], k[j]))
             for j in range(vis[i])]
        if not s:
            continue
        m = max(s)
        e = [math.exp(x - m) for x in s]
        tot = math.fsum(e)
        for j in range(vis[i]):
            p[i][j] = e[j] / tot
    return np.array(p)


def _probs_drop_scale(q, k, scale, vis):
    return oa.softmax_probs_ref(q, k, 1.0, vis)


def _probs_base_two(q, k, scale, vis):
    # exp2 in place of exp: the scores scaled by ln 2 give the same as base 2
    return oa.softmax_probs_ref(q, k, scale * math.log(2.0), vis)


def _probs_no_mask(q, k, scale, vis):
    return oa.softmax_probs_ref(q, k, scale, [len(k)] * len(q))


@pytest.mark.parametrize("mutant", [None, _probs_drop_scale, _probs_base_two, _probs_no_mask])
def test_softmax_probs_match_brute_force_and_weight_the_values(mutant):
    """The probabilities equal a pure-Python softmax of the scaled scores, P V is
    attend_rows' output and log sum exp of the scaled visible scores its lse; each
    planted mistake (scale dropped, base 2, mask ignored) fails the brute force."""
    rng = np.random.default_rng(61)
    q, k, v = rng.standard_normal((5, 6)), rng.standard_normal((13, 6)), rng.standard_normal((13, 4))
    vis, scale = [13, 1, 0, 7, 12], 0.37
    fn = oa.softmax_probs_ref if mutant is None else mutant
    p = fn(q, k, scale, vis)
    ref = _brute_probs(q, k, scale, vis)
    if mutant is not None:
        assert np.abs(p - ref).max() > 1e-6
        return
    assert np.abs(p - ref).max() < 1e-14
    o, lse = oracle.attend_rows(q, k, v, scale, vis)
    assert np.abs(p @ v - o).max() < 1e-13
    for i, n in enumerate(vis):
        s = [scale * math.fsum(float(a) * float(b) for a, b in zip(q[i], k[j])) for j in range(n)]
        if not s:
            assert lse[i] == -np.inf and (p[i] == 0).all()
            continue
        m = max(s)
        assert abs(lse[i] - (m + math.log(math.fsum(math.exp(x - m) for x in s)))) < 1e-13


def test_page_permutation_leaves_output_unchanged():
    case = make_case("p", seq_lens=[40, 17, 64], Hq=4, Hkv=2, D=8, page_size=16, seed=8,
                     num_pages=12)
    o1, l1 = run_oracle(case)
    perm = np.random.default_rng(0).permutation(12)          # new page id of old page i
    inv = np.argsort(perm)
    kp, vp = bits(case.k_pool), bits(case.v_pool)
    bt = case.block_tables.numpy().copy()
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1)
    o2, l2 = oracle.attention_ref(bits(case.q), kp[inv], vp[inv], bt2, case.seq_lens_k.numpy(),
                                  case.cu_seqlens_q.numpy(), case.scale, False, 16)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_page_size_does_not_change_the_result():
    a = make_case("a", seq_lens=[100, 65], Hq=4, Hkv=2, D=8, page_size=16, seed=9, permute=False)
    ka, va = oracle.gather_sequence_kv, None
    # rebuild the same logical KV in a 64-token page pool
    kp16, vp16 = bits(a.k_pool), bits(a.v_pool)
    bt = a.block_tables.numpy()
    lens = a.seq_lens_k.numpy()
    pools = []
    for pool in (kp16, vp16):
        seqs = [pool[bt[b, :-(-lens[b] // 16)]].reshape(-1, 2, 8)[:lens[b]] for b in range(2)]
        big = np.zeros((4, 64, 2, 8), dtype=np.uint16)
        for b, s in enumerate(seqs):
            flat = np.zeros((128, 2, 8), dtype=np.uint16)
            flat[:len(s)] = s
            big[2 * b:2 * b + 2] = flat.reshape(2, 64, 2, 8)
        pools.append(big)
    bt64 = np.array([[0, 1], [2, 3]], dtype=np.int32)
    o16, l16 = run_oracle(a)
    o64, l64 = oracle.attention_ref(bits(a.q), pools[0], pools[1], bt64, lens,
                                    a.cu_seqlens_q.numpy(), a.scale, False, 64)
    assert np.array_equal(o16, o64) and np.array_equal(l16, l64)


def test_gqa_equals_mha_with_repeated_kv():
    case = make_case("g", seq_lens=[33, 70], q_lens=[3, 5], Hq=6, Hkv=2, D=8, page_size=16,
                     seed=10, causal=True)
    o, l = run_oracle(case)
    kp, vp = bits(case.k_pool), bits(case.v_pool)
    kr, vr = np.repeat(kp, 3, axis=2), np.repeat(vp, 3, axis=2)
    o2, l2 = oracle.attention_ref(bits(case.q), kr, vr, case.block_tables.numpy(),
                                  case.seq_lens_k.numpy(), case.cu_seqlens_q.numpy(),
                                  case.scale, True, 16)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


@pytest.mark.parametrize("tile", [1, 7, 16, 64, 97])
def test_tiled_online_softmax_equals_untiled(tile):
    rng = np.random.default_rng(tile)
    q, k, v = rng.standard_normal((6, 16)) * 3, rng.standard_normal((97, 16)), \
        rng.standard_normal((97, 16))
    vis = [97, 1, 50, 0, 64, 33]
    o, lse = oracle.attend_rows(q, k, v, 0.25, vis)
    ot, lset = oracle.tiled_attend_rows(q, k, v, 0.25, vis, tile)
    assert_close(ot, o, 1e-12)
    assert_close(lset, lse, 1e-12)


@pytest.mark.parametrize("bounds", [[0, 97], [0, 32, 64, 97], [0, 0, 5, 5, 97],
                                    [0, 1, 2, 3, 50, 97, 97, 97], [0, 40, 80, 97]])
@pytest.mark.parametrize("visible", [97, 45, 1, 0])
def test_split_and_merge_equals_unsplit(bounds, visible):
    rng = np.random.default_rng(len(bounds) * 100 + visible)
    q, k, v = rng.standard_normal(16), rng.standard_normal((97, 16)), rng.standard_normal((97, 16))
    o, lse = oracle.attend_rows(q[None], k, v, 0.3, [visible])
    oc, lc = oracle.split_partials_ref(q, k, v, 0.3, visible, bounds)
    om, lm = oracle.merge_ref(oc, lc)
    assert_close(om, o[0], 1e-12)
    assert_close(np.atleast_1d(lm), lse, 1e-12)


def test_merge_of_all_empty_chunks_is_zero():
    o, l = oracle.merge_ref(np.ones((3, 4)), np.full(3, -np.inf))
    assert (o == 0).all() and l == -np.inf


def test_last_causal_row_equals_decode_of_the_same_sequence():
    pre = make_case("c", seq_lens=[57], q_lens=[57], Hq=4, Hkv=1, D=8, page_size=16, seed=11,
                    causal=True)
    o, l = run_oracle(pre)
    dec_q = pre.q[-1:].clone()
    o2, l2 = oracle.attention_ref(bits(dec_q), bits(pre.k_pool), bits(pre.v_pool),
                                  pre.block_tables.numpy(), pre.seq_lens_k.numpy(),
                                  np.array([0, 1]), pre.scale, False, 16)
    assert_close(o[-1], o2[0])          # BLAS may round a 1-row product differently
    assert_close(l[-1], l2[0])


def test_chunked_prefill_equals_one_shot():
    full = make_case("f", seq_lens=[80], q_lens=[80], Hq=2, Hkv=1, D=8, page_size=16, seed=12,
                     causal=True)
    o, l = run_oracle(full)
    args = (bits(full.k_pool), bits(full.v_pool), full.block_tables.numpy())
    qb = bits(full.q)
    # first chunk: 30 queries over a 30-key prefix; second: 50 queries over all 80 keys
    o1, l1 = oracle.attention_ref(qb[:30], *args, np.array([30]), np.array([0, 30]),
                                  full.scale, True, 16)
    o2, l2 = oracle.attention_ref(qb[30:], *args, np.array([80]), np.array([0, 50]),
                                  full.scale, True, 16)
    assert_close(np.concatenate([o1, o2]), o)
    assert_close(np.concatenate([l1, l2]), l)


def test_rows_ref_matches_full_ref():
    case = make_case("r", hist_lens=[20, 0, 45], q_lens=[5, 16, 1], write_new=True, causal=True,
                     Hq=4, Hkv=2, D=8, page_size=16, seed=13)
    kp, vp = oracle.kv_write_ref(bits(case.k_pool), bits(case.v_pool), bits(case.k_new),
                                 bits(case.v_new), case.cu_new.numpy(), case.start_pos.numpy(),
                                 case.block_tables.numpy(), 16)
    args = (bits(case.q), kp, vp, case.block_tables.numpy(), case.seq_lens_k.numpy(),
            case.cu_seqlens_q.numpy(), case.scale, True, 16)
    o, l = oracle.attention_ref(*args)
    rows = [(0, 0), (4, 3), (5, 1), (20, 2), (21, 0)]
    orow, lrow = oracle.attention_rows_ref(*args, rows=rows)
    for i, (t, h) in enumerate(rows):
        assert_close(orow[i], o[t, h])
        assert_close(lrow[i], l[t, h])


# ----------------------------------------------------------------------------
# page writes
# ----------------------------------------------------------------------------

def test_kv_write_matches_a_loop_and_round_trips():
    case = make_case("w", hist_lens=[0, 13, 40], q_lens=[20, 3, 1], write_new=True, Hq=4, Hkv=2,
                     D=8, page_size=16, seed=14, num_pages=10)
    kp, vp = bits(case.k_pool), bits(case.v_pool)
    kn, vn = bits(case.k_new), bits(case.v_new)
    bt = case.block_tables.numpy()
    cu, sp = case.cu_new.numpy(), case.start_pos.numpy()
    ko, vo = oracle.kv_write_ref(kp, vp, kn, vn, cu, sp, bt, 16)
    kl, vl = kp.copy(), vp.copy()
    for b in range(3):
        for t in range(cu[b], cu[b + 1]):
            pos = sp[b] + t - cu[b]
            kl[bt[b][pos // 16], pos % 16] = kn[t]
            vl[bt[b][pos // 16], pos % 16] = vn[t]
    assert np.array_equal(ko, kl) and np.array_equal(vo, vl)
    assert np.array_equal(kp, bits(case.k_pool))                  # input untouched
    for b in range(3):
        L = int(case.seq_lens_k[b])
        g = oracle.gather_sequence_kv(ko, bt[b], L, 16)
        new = oracle.bf16_bits_to_f64(kn[cu[b]:cu[b + 1]])
        assert np.array_equal(g[sp[b]:], new)
        assert np.isfinite(g).all()                               # every NaN slot was written


# ----------------------------------------------------------------------------
# traffic figures printed by the pages
# ----------------------------------------------------------------------------

def test_traffic_figures_from_the_pages():
    with open(os.path.join(GOLDEN, "traffic_figures.json")) as f:
        entries = json.load(f)["entries"]
    e = entries
    assert units.kv_bytes_per_head(e[0]["seq_len"], e[0]["head_dim"], e[0]["elem_bytes"]) == e[0]["bytes"]
    assert units.score_matrix_bytes(e[1]["n"], e[1]["n"], e[1]["elem_bytes"]) == e[1]["bytes"]
    assert units.naive_attention_traffic(e[2]["n"], e[2]["elem_bytes"], e[2]["passes"]) == e[2]["bytes"]
    assert units.score_matrix_bytes(e[3]["n_q"], e[3]["n_k"], e[3]["elem_bytes"]) == e[3]["bytes"]
    assert units.score_matrix_bytes(e[4]["n"], e[4]["n"], e[4]["elem_bytes"]) == e[4]["bytes"]
    assert e[2]["bytes"] // e[0]["bytes"] == e[5]["ratio"]
    # one sequence, one head, no query/output/table overhead: the decode unit is the same 2 MiB
    one = units.decode_bytes([4096], 1, 1, 128, 16) - 2 * 128 * 2 - 256 * 4 - 4
    assert one == e[0]["bytes"]


def test_workload_units_at_the_five_sizes():
    assert units.decode_bytes([17, 64, 100, 255], 8, 2, 64, 16) == 231_556
    assert units.decode_bytes([8192] * 32, 28, 4, 128, 16) == 537_395_328
    assert units.decode_bytes([131072] * 8, 64, 8, 128, 64) == 4_295_295_008
    assert units.prefill_flops([4096] * 4, [4096] * 4, 32, 128, True) == 549_890_031_616
    # brute-force pair count on a small ragged causal batch
    lens, ql = [7, 3, 12], [7, 1, 5]
    pairs = sum(max(0, L - n + i + 1) for L, n in zip(lens, ql) for i in range(n))
    assert units.prefill_pairs(lens, ql, True) == pairs
    assert units.prefill_pairs(lens, ql, False) == sum(L * n for L, n in zip(lens, ql))


# ----------------------------------------------------------------------------
# planted mistakes: each must be caught by a pin above
# ----------------------------------------------------------------------------

def _mut_drop_scale(q_rows, k, v, scale, visible, *rest):
    return _orig_attend(q_rows, k, v, 1.0, visible, *rest)


def _mut_no_mask(q_rows, k, v, scale, visible, *rest):
    return _orig_attend(q_rows, k, v, scale, np.full(len(np.atleast_1d(visible)), k.shape[0]))


def _mut_off_by_one_causal(q_rows, k, v, scale, visible, *rest):
    vis = np.asarray(visible) - 1
    return _orig_attend(q_rows, k, v, scale, np.maximum(vis, 0), *rest)


def _mut_transposed_value(q_rows, k, v, scale, visible, *rest):
    o, l = _orig_attend(q_rows, k, v, scale, visible, *rest)
    return o[:, ::-1].copy(), l


_orig_attend = oa.attend_rows


@pytest.mark.parametrize("mutant", [_mut_drop_scale, _mut_no_mask, _mut_off_by_one_causal,
                                    _mut_transposed_value])
def test_planted_oracle_mistakes_are_caught(monkeypatch, mutant):
    case = make_case("m", seq_lens=[20, 9], q_lens=[4, 2], Hq=2, Hkv=1, D=4, page_size=3,
                     seed=15, causal=True)
    ob, lb = brute_attention(case)
    monkeypatch.setattr(oa, "attend_rows", mutant)
    o, l = run_oracle(case)
    with pytest.raises(AssertionError):
        assert_close(o, ob)
        assert_close(l, lb)


def test_planted_gqa_mapping_mistake_is_caught(monkeypatch):
    case = make_case("m", seq_lens=[20], Hq=4, Hkv=2, D=4, page_size=4, seed=16)
    ob, _ = brute_attention(case)
    # a wrong head mapping (h % Hkv instead of h // G) through a patched gather
    orig = oa.gather_sequence_kv

    def swapped(pool, row, L, ps):
        g = orig(pool, row, L, ps)
        return g[:, ::-1]
    monkeypatch.setattr(oa, "gather_sequence_kv", swapped)
    o, _ = run_oracle(case)
    assert np.abs(o - ob).max() > 1e-3


def test_planted_merge_mistake_is_caught(monkeypatch):
    rng = np.random.default_rng(17)
    q, k, v = rng.standard_normal(8), rng.standard_normal((40, 8)), rng.standard_normal((40, 8))
    o, _ = oracle.attend_rows(q[None], k, v, 1.0, [40])
    oc, lc = oracle.split_partials_ref(q, k, v, 1.0, 40, [0, 10, 40])
    # forgetting the lse weights (plain average of chunk outputs) must not pass
    assert np.abs(oc.mean(axis=0) - o[0]).max() > 1e-3
    om, _ = oracle.merge_ref(oc, lc)
    assert np.abs(om - o[0]).max() < 1e-12


# ----------------------------------------------------------------------------
# sliding window (R4)
# ----------------------------------------------------------------------------

def _window_case(window, causal=True, seed=31):
    return make_case("win", seq_lens=[40, 7, 23], q_lens=[6, 7, 1], Hq=4, Hkv=2, D=8,
                     page_size=3, seed=seed, causal=causal, window=window)


def test_window_of_one_returns_each_rows_own_value_row():
    """Causal window 1: a row sees only the key at its own position, so O is that
    key's value row exactly and lse is its scaled score."""
    case = _window_case(1)
    o, lse = run_oracle(case)
    q, kp, vp = bits(case.q), bits(case.k_pool), bits(case.v_pool)
    bt, cu = case.block_tables.numpy(), case.cu_seqlens_q.numpy()
    for b, L in enumerate(case.seq_lens):
        n = int(cu[b + 1] - cu[b])
        for i in range(n):
            pos = L - n + i
            page, slot = int(bt[b][pos // 3]), pos % 3
            for h in range(4):
                kv = oracle.bf16_bits_to_f64(kp[page, slot, h // 2])
                vv = oracle.bf16_bits_to_f64(vp[page, slot, h // 2])
                qv = oracle.bf16_bits_to_f64(q[int(cu[b]) + i, h])
                assert np.array_equal(o[int(cu[b]) + i, h], vv)
                assert abs(lse[int(cu[b]) + i, h] - case.scale * float(qv @ kv)) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_window_covering_every_key_changes_nothing(causal):
    case = _window_case(0, causal)
    o0, l0 = run_oracle(case)
    o1, l1 = run_oracle(case, window=41)       # longer than every sequence
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


@pytest.mark.parametrize("window,causal", [(1, True), (4, True), (9, False), (40, True)])
def test_window_matches_brute_force(window, causal):
    case = _window_case(window, causal)
    o, l = run_oracle(case)
    ob, lb = brute_attention(case)
    assert_close(o, ob)
    assert_close(l, lb)


def test_window_equals_attention_over_the_sliced_keys():
    """A windowed row is plain attention over keys p - w + 1 .. p (no mask at all)."""
    case = _window_case(5)
    o, _ = run_oracle(case)
    q, bt = bits(case.q), case.block_tables.numpy()
    L, n = case.seq_lens[0], 6
    k = oa.gather_sequence_kv(bits(case.k_pool), bt[0], L, 3)[:, 1]
    v = oa.gather_sequence_kv(bits(case.v_pool), bt[0], L, 3)[:, 1]
    for i in range(n):
        pos = L - n + i
        lo = max(0, pos - 4)
        qi = oracle.bf16_bits_to_f64(q[i, 2])[None]
        os_, _ = oracle.attend_rows(qi, k[lo:pos + 1], v[lo:pos + 1], case.scale, [pos + 1 - lo])
        assert np.abs(os_[0] - o[i, 2]).max() < 1e-12


@pytest.mark.parametrize("mutant", ["off_by_one", "ignored"])
def test_planted_window_mistakes_are_caught(monkeypatch, mutant):
    case = _window_case(4)
    ob, lb = brute_attention(case)
    real = oa._first_visible
    if mutant == "off_by_one":
        monkeypatch.setattr(oa, "_first_visible",
                            lambda L, n, w: np.maximum(0, real(L, n, w) - 1))
    else:
        monkeypatch.setattr(oa, "_first_visible", lambda L, n, w: real(L, n, 0))
    o, _ = run_oracle(case)
    assert np.abs(o - ob).max() > 1e-6


# ----------------------------------------------------------------------------
# ALiBi (R5)
# ----------------------------------------------------------------------------

SLOPES = np.array([0.5, 0.25, 0.125, 0.0625])


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 9)])
def test_alibi_matches_brute_force(causal, window):
    case = _window_case(window, causal, seed=44)
    o, l = run_oracle(case, alibi=SLOPES)
    ob, lb = brute_attention(case, alibi=SLOPES)
    assert_close(o, ob)
    assert_close(l, lb)


def test_alibi_with_zero_query_gives_geometric_weights():
    """q = 0: every score is the bias alone, so a causal row at position p weights key
    j by exp(-s (p - j)) / sum_i exp(-s (p - i)), a geometric series in closed form."""
    case = make_case("ag", seq_lens=[30], q_lens=[1], Hq=2, Hkv=1, D=4, page_size=4, seed=2,
                     causal=True)
    case.q = torch.zeros_like(case.q)
    slopes = np.array([0.3, 1.1])
    o, lse = run_oracle(case, alibi=slopes)
    v = oa.gather_sequence_kv(bits(case.v_pool), case.block_tables.numpy()[0], 30, 4)[:, 0]
    for h, s_ in enumerate(slopes):
        r = math.exp(-s_)
        w = np.array([r ** (29 - j) for j in range(30)])
        den = (1 - r ** 30) / (1 - r)                      # sum of r^k, k = 0..29
        assert abs(w.sum() - den) < 1e-12
        assert np.abs(o[0, h] - (w @ v) / den).max() < 1e-12
        assert abs(lse[0, h] - math.log(den)) < 1e-12


def test_alibi_is_a_shift_of_a_position_independent_bias():
    """slope * (j - p) differs from slope * j by a per-row constant: the same O, and
    lse lower by slope * p."""
    case = _window_case(0, True, seed=45)
    o1, l1 = run_oracle(case, alibi=SLOPES)
    q, kp, vp, bt = bits(case.q), bits(case.k_pool), bits(case.v_pool), case.block_tables.numpy()
    cu = case.cu_seqlens_q.numpy()
    for b, L in enumerate(case.seq_lens):
        n = int(cu[b + 1] - cu[b])
        k = oa.gather_sequence_kv(kp, bt[b], L, 3)
        v = oa.gather_sequence_kv(vp, bt[b], L, 3)
        for h in range(4):
            rows = oracle.bf16_bits_to_f64(q[int(cu[b]):int(cu[b]) + n, h])
            vis = L - n + np.arange(n) + 1
            o0, l0 = oracle.attend_rows(rows, k[:, h // 2], v[:, h // 2], case.scale, vis, None,
                                        SLOPES[h], np.zeros(n))
            pos = L - n + np.arange(n)
            assert np.abs(o0 - o1[int(cu[b]):int(cu[b]) + n, h]).max() < 1e-12
            assert np.abs(l0 - SLOPES[h] * pos - l1[int(cu[b]):int(cu[b]) + n, h]).max() < 1e-9


@pytest.mark.parametrize("mutant", ["sign", "scaled"])
def test_planted_alibi_mistakes_are_caught(mutant):
    case = _window_case(0, True, seed=46)
    ob, _ = brute_attention(case, alibi=SLOPES)
    wrong = -SLOPES if mutant == "sign" else SLOPES * case.scale
    o, _ = run_oracle(case, alibi=wrong)
    assert np.abs(o - ob).max() > 1e-6


@pytest.mark.parametrize("split_kv_heads", [False, True])
@pytest.mark.parametrize("causal,window,alibi", [(True, 0, False), (False, 0, False),
                                                 (True, 5, True), (True, 0, True)])
def test_per_sequence_oracle_helper_equals_the_whole_pool_oracle(split_kv_heads, causal,
                                                                 window, alibi):
    """The full-size parity tests run the oracle one sequence (and KV head) at a time
    on the sequence's own pages; that must be the oracle over the whole pool, bit for
    bit, including empty sequences, chunks over history and rows before the first key."""
    from tests.parity import oracle_by_sequence, oracle_full
    case = make_case("bys", seq_lens=[40, 0, 17, 65], q_lens=[3, 2, 20, 65], Hq=6, Hkv=2, D=8,
                     page_size=4, seed=71, causal=causal, window=window, num_pages=40)
    slopes = np.array([0.3, -0.1, 0.05, 0.0, 0.2, 0.7]) if alibi else None
    kp, vp = bits(case.k_pool), bits(case.v_pool)
    o1, l1 = oracle_full(case, kp, vp, alibi=slopes)
    o2, l2 = oracle_by_sequence(case, kp, vp, split_kv_heads=split_kv_heads, alibi=slopes)
    assert np.array_equal(o1, o2)
    assert np.array_equal(l1, l2)


# ----------------------------------------------------------------------------
# document masks (R6)
# ----------------------------------------------------------------------------

def _doc_case(causal=True, seed=91, window=0):
    lens, ql = [40, 23, 0, 31], [7, 23, 3, 40]
    case = make_case("doc", seq_lens=lens, q_lens=ql, Hq=4, Hkv=2, D=8, page_size=4,
                     seed=seed, causal=causal, window=window,
                     num_pages=sum(-(-L // 4) for L in lens) + 2)
    return case, document_ranges(lens, ql, 4, seed)


@pytest.mark.parametrize("causal,window,alibi", [(True, 0, False), (False, 0, False),
                                                 (True, 6, False), (True, 0, True),
                                                 (False, 5, True)])
def test_document_ranges_match_brute_force(causal, window, alibi):
    case, kr = _doc_case(causal, window=window)
    slopes = np.array([0.25, -0.1, 0.5, 0.0]) if alibi else None
    o, lse = run_oracle(case, alibi=slopes, key_ranges=kr)
    ob, lb = brute_attention(case, alibi=slopes, key_ranges=kr)
    assert_close(o, ob)
    assert_close(lse, lb)
    # some rows keep only part of their causal keys, some see nothing (before the
    # first key of their sequence)
    assert np.isneginf(lse).any() and np.isfinite(lse).any()


def test_document_row_equals_attention_over_its_documents_keys():
    """A row of document [s, e) equals unmasked attention over that document's keys
    alone (the slice s .. min(e, p + 1) for a causal row at position p)."""
    case, (lo, hi) = _doc_case(True, seed=92)
    o, lse = run_oracle(case, key_ranges=(lo, hi))
    q = oracle.bf16_bits_to_f64(bits(case.q))
    cu = case.cu_seqlens_q.numpy()
    for b, L in enumerate(case.seq_lens):
        k = oracle.gather_sequence_kv(bits(case.k_pool), case.block_tables[b].numpy(), L, 4)
        v = oracle.gather_sequence_kv(bits(case.v_pool), case.block_tables[b].numpy(), L, 4)
        n = int(cu[b + 1] - cu[b])
        for i in range(n):
            t, p = int(cu[b]) + i, L - n + i
            s0, s1 = int(lo[t]), min(int(hi[t]), p + 1)
            for h in range(case.Hq):
                if s1 <= s0:
                    assert np.isneginf(lse[t, h]) and (o[t, h] == 0).all()
                    continue
                ks, vs = k[s0:s1, h // 2], v[s0:s1, h // 2]
                s = case.scale * ks @ q[t, h]
                w = np.exp(s - s.max())
                assert np.abs(o[t, h] - w @ vs / w.sum()).max() < 1e-12
                assert abs(lse[t, h] - (s.max() + np.log(w.sum()))) < 1e-12


def test_one_document_per_sequence_changes_nothing():
    case, _ = _doc_case(True, seed=93)
    kr = document_ranges(case.seq_lens, case.q_lens, 1, 93)
    o1, l1 = run_oracle(case)
    o2, l2 = run_oracle(case, key_ranges=kr)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("mutant,causal", [("hi_inclusive", False), ("lo_ignored", True),
                                           ("lo_off_by_one", True), ("lo_ignored", False)])
def test_planted_document_mistakes_are_caught(mutant, causal):
    """(A causal row's own position lies in its document, so key_hi binds only
    without the causal mask.)"""
    case, (lo, hi) = _doc_case(causal, seed=94)
    ob, lb = brute_attention(case, key_ranges=(lo, hi))
    if mutant == "hi_inclusive":
        kr = (lo, hi + 1)
    elif mutant == "lo_ignored":
        kr = (np.zeros_like(lo), hi)
    else:
        kr = (lo + 1, hi)
    o, l = run_oracle(case, key_ranges=kr)
    with pytest.raises(AssertionError):
        assert_close(o, ob)
        assert_close(l, lb)


def test_document_ranges_layout():
    """The generator's ranges: each row's range holds its own position (rows at
    negative positions get an empty range), ranges tile every sequence."""
    lens, ql = [50, 9, 0, 300], [10, 9, 2, 1]
    lo, hi = document_ranges(lens, ql, 5, 7)
    t = 0
    for L, n in zip(lens, ql):
        for i in range(n):
            p = L - n + i
            if p < 0:
                assert lo[t] == hi[t] == 0
            else:
                assert 0 <= lo[t] <= p < hi[t] <= L
            t += 1


# ----------------------------------------------------------------------------
# general masks (R7): a predicate of (sequence, head, query index, key index), and
# its block form
# ----------------------------------------------------------------------------

def _mask_case(causal=False, seed=71):
    return make_case("msk", seq_lens=[150, 70, 0, 131], q_lens=[130, 9, 0, 131], Hq=4, Hkv=2,
                     D=8, page_size=16, seed=seed, causal=causal)


def _run_mask(case, mask_fn, causal=None, window=0, key_ranges=None):
    return oracle.attention_ref(bits(case.q), bits(case.k_pool), bits(case.v_pool),
                                case.block_tables.numpy(), case.seq_lens_k.numpy(),
                                case.cu_seqlens_q.numpy(), case.scale,
                                case.causal if causal is None else causal, case.page_size,
                                window, None, key_ranges, mask_fn)


def _lens(case):
    cu = case.cu_seqlens_q.numpy()
    return case.seq_lens_k.numpy(), cu[1:] - cu[:-1]


def test_mask_fn_that_allows_everything_changes_nothing():
    case = _mask_case(causal=True)
    o0, l0 = _run_mask(case, None)
    o1, l1 = _run_mask(case, lambda b, h, q, k: np.ones(np.broadcast(q, k).shape, bool))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_mask_fn_reproduces_causal_window_and_documents():
    """The causal bound (R2), the window (R4) and document ranges (R6) written as
    predicates give the same bits as the built-in forms."""
    case = _mask_case()
    L, n = _lens(case)
    causal_fn = lambda b, h, q, k: k <= L[b] - n[b] + q
    assert_close(_run_mask(case, causal_fn, causal=False)[0], _run_mask(case, None, True)[0], 0)
    w = 20
    win_fn = lambda b, h, q, k: (k <= L[b] - n[b] + q) & (k > L[b] - n[b] + q - w)
    o_w, l_w = _run_mask(case, win_fn, causal=False)
    o_r, l_r = _run_mask(case, None, causal=True, window=w)
    assert_close(o_w, o_r, 0)
    assert_close(l_w, l_r, 0)
    kr = document_ranges(list(L), list(n), 3, 5)
    cu = case.cu_seqlens_q.numpy()
    doc_fn = lambda b, h, q, k: (k >= kr[0][cu[b] + q]) & (k < kr[1][cu[b] + q])
    o_d, l_d = _run_mask(case, doc_fn, causal=True)
    o_k, l_k = _run_mask(case, None, causal=True, key_ranges=kr)
    assert_close(o_d, o_k, 0)
    assert_close(l_d, l_k, 0)


def _head_parity(b, h, q, k):
    # even heads see even keys only, odd heads every key up to 3 q + 5: depends on
    # every argument, so a predicate wired to the wrong one shows
    return np.where(np.asarray(h) % 2 == 0, np.asarray(k) % 2 == 0,
                    np.asarray(k) <= 3 * np.asarray(q) + 5 + np.asarray(b))


@pytest.mark.parametrize("causal", [False, True])
def test_mask_fn_matches_brute_force(causal):
    case = make_case("mbf", seq_lens=[23, 9, 0, 17], q_lens=[5, 9, 0, 3], Hq=4, Hkv=2, D=4,
                     page_size=3, seed=3, causal=causal)
    ob, lb = brute_attention(case, pred=_head_parity)
    oo, lo = _run_mask(case, _head_parity)
    assert_close(oo, ob, 1e-12)
    assert_close(lo, lb, 1e-12)


def _random_block_map(case, seed, density=0.5, block=64):
    L, n = _lens(case)
    rng = np.random.default_rng(seed)
    qb = max(1, -(-int(n.max()) // block))
    kb = max(1, -(-int(L.max()) // block))
    return (rng.random((len(L), qb, kb)) < density).astype(np.uint8)


@pytest.mark.parametrize("causal", [False, True])
def test_block_map_matches_brute_force(causal):
    """A block map at 8 x 8 blocks on a small case against the brute force, whose
    predicate looks the entries up one by one."""
    case = make_case("mbm", seq_lens=[30, 19, 26], q_lens=[17, 19, 2], Hq=2, Hkv=1, D=4,
                     page_size=16, seed=9, causal=causal)
    bm = _random_block_map(case, 4, 0.6, block=8)
    pred = lambda b, h, i, j: (i // 8 < bm.shape[1] and j // 8 < bm.shape[2]
                               and bm[b][i // 8][j // 8] != 0)
    ob, lb = brute_attention(case, pred=pred)
    oo, lo = _run_mask(case, oracle.block_map_mask(bm, block=8))
    assert_close(oo, ob, 1e-12)
    assert_close(lo, lb, 1e-12)


def test_block_map_edges():
    """All blocks visible = no map; no block visible = every row sees nothing (O = 0,
    lse = -inf); a map too small for the sequence hides the keys outside it."""
    case = _mask_case(causal=True)
    ones = np.ones_like(_random_block_map(case, 1))
    o0, l0 = _run_mask(case, None)
    o1, l1 = _run_mask(case, oracle.block_map_mask(ones))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    o2, l2 = _run_mask(case, oracle.block_map_mask(np.zeros_like(ones)))
    assert not o2.any() and np.all(l2 == -np.inf)
    small = ones[:, :1, :1]                 # rows 0..63, keys 0..63 only
    o3, l3 = _run_mask(case, oracle.block_map_mask(small))
    L, n = _lens(case)
    cu = case.cu_seqlens_q.numpy()
    ref = oracle.attention_ref(bits(case.q), bits(case.k_pool), bits(case.v_pool),
                               case.block_tables.numpy(), np.minimum(L, 64), cu, case.scale,
                               False, case.page_size)
    for b in range(len(L)):
        for i in range(int(n[b])):
            t = int(cu[b]) + i
            if i >= 64 or L[b] == 0:
                assert not o3[t].any() and np.all(l3[t] == -np.inf)
            elif L[b] - n[b] + i >= 63:
                # the causal bound lies past key 63: the row sees keys 0..63
                assert_close(o3[t], ref[0][t], 1e-12)


@pytest.mark.parametrize("mutant", ["transposed", "position"])
def test_planted_mask_mistakes_are_caught(mutant):
    """A block map read transposed, or indexed by absolute position instead of the
    row's index in its query run, fails the brute force."""
    case = make_case("mmu", seq_lens=[40, 33], q_lens=[12, 20], Hq=2, Hkv=1, D=4,
                     page_size=16, seed=2, causal=False)
    bm = _random_block_map(case, 8, 0.5, block=8)
    bm = np.concatenate([bm, np.ones((bm.shape[0], max(0, bm.shape[2] - bm.shape[1]),
                                      bm.shape[2]), np.uint8)], axis=1)
    pred = lambda b, h, i, j: (i // 8 < bm.shape[1] and j // 8 < bm.shape[2]
                               and bm[b][i // 8][j // 8] != 0)
    ob, _ = brute_attention(case, pred=pred)
    L, n = _lens(case)
    if mutant == "transposed":
        bad = np.ascontiguousarray(np.swapaxes(bm, 1, 2))
        fn = oracle.block_map_mask(bad, block=8)
    else:
        good = oracle.block_map_mask(bm, block=8)
        fn = lambda b, h, q, k: good(b, h, q + (L[b] - n[b]), k)
    oo, _ = _run_mask(case, fn)
    assert not np.allclose(oo, ob, atol=1e-6)


def test_rows_ref_with_mask_fn_matches_full_ref():
    case = _mask_case(causal=True)
    bm = _random_block_map(case, 6, 0.5)
    fn = oracle.block_map_mask(bm)
    o, l = _run_mask(case, fn)
    rows = [(0, 0), (64, 1), (129, 3), (130, 2), (138, 0), (139, 1), (200, 3), (269, 2)]
    ro, rl = oracle.attention_rows_ref(bits(case.q), bits(case.k_pool), bits(case.v_pool),
                                       case.block_tables.numpy(), case.seq_lens_k.numpy(),
                                       case.cu_seqlens_q.numpy(), case.scale, True,
                                       case.page_size, rows, mask_fn=fn)
    for i, (t, h) in enumerate(rows):
        assert_close(ro[i], o[t, h], 1e-12)
        assert_close(rl[i], l[t, h], 1e-12)


def test_block_map_pair_count_matches_a_loop():
    """units.block_map_pairs (the flop count of a prefill with a block map) against
    a loop over every (row, key) of small ragged cases, 16 x 16 blocks."""
    rng = np.random.default_rng(0)
    for _ in range(6):
        lens = rng.integers(0, 120, 3).tolist()
        ql = [int(min(L, rng.integers(1, 90))) if L else 0 for L in lens]
        bm = (rng.random((3, 5, 7)) < 0.5).astype(np.uint8)
        for causal in (False, True):
            n_pairs = sum(1 for b in range(3) for i in range(ql[b]) for j in range(lens[b])
                          if not (causal and j > lens[b] - ql[b] + i)
                          and i // 16 < 5 and j // 16 < 7 and bm[b, i // 16, j // 16])
            assert units.block_map_pairs(lens, ql, causal, bm, 16) == n_pairs
