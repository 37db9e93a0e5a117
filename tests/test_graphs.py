"""A whole serving step captured in one HIP graph.

The step writes new tokens into bf16 and FP8 pools, runs a key-split prefill, a
general prefill (sliding window plus ALiBi), a bf16 decode and an FP8 decode.  The
graph is replayed several times, with eager calls of other shapes that reuse the
same workspaces between the replays; every replay must reproduce the eager results
bit for bit (outputs, log-sum-exps and the written pools).  No call in the step
records a memset or allocates, so the step is capturable as it stands.
"""

import numpy as np
import pytest
import torch

import paged_kv_flashattention_amd as pa
from tests.parity import as_f64, assert_lse, assert_parity, oracle_full, pools_after_write
from workloads import bits, make_case, random_e4m3_codes

pytestmark = pytest.mark.gpu

K_SCALE, V_SCALE = 0.0625, 0.03125


def _cases():
    pf = make_case("gpf", hist_lens=[3000, 0, 200], q_lens=[300, 129, 64], write_new=True,
                   causal=True, Hq=8, Hkv=2, D=128, page_size=16, seed=70, device="cuda")
    dc = make_case("gdc", hist_lens=[4000, 17, 900, 0], q_lens=[1, 1, 1, 1], write_new=True,
                   causal=True, Hq=28, Hkv=4, D=128, page_size=16, seed=71, device="cuda")
    return pf, dc


class Step:
    """Preallocated buffers and the step's launches (no allocation inside run())."""

    def __init__(self, pf, dc):
        self.pf, self.dc = pf, dc
        dev = "cuda"
        shape = tuple(dc.k_pool.shape)
        self.kc = random_e4m3_codes(shape, 72, dev)
        self.vc = random_e4m3_codes(shape, 73, dev)
        self.slopes = torch.tensor([2.0 ** (-(i + 1)) for i in range(pf.Hq)],
                                   dtype=torch.float32, device=dev)
        self.pf_splits = 4
        pf_ws = pa.prefill_workspace_bytes(pf.B, pf.q.shape[0], pf.max_q_len, pf.Hq, pf.D,
                                           self.pf_splits)
        # large enough for the other-shape calls made between replays as well
        pf_ws = max(pf_ws, pa.prefill_workspace_bytes(1, 700, 700, 8, 128, 2), 1)
        self.pf_ws = torch.empty(pf_ws, dtype=torch.uint8, device=dev)
        self.dc_splits = 4
        dc_ws = pa.decode_workspace_bytes(dc.B, dc.Hq, dc.Hkv, dc.D, 8192, self.dc_splits)
        self.dc_ws = torch.empty(dc_ws, dtype=torch.uint8, device=dev)
        self.dc8_ws = torch.empty(dc_ws, dtype=torch.uint8, device=dev)
        Tq = pf.q.shape[0]
        self.bufs = {
            "pf_o": torch.empty((Tq, pf.Hq, pf.D), dtype=torch.bfloat16, device=dev),
            "pf_l": torch.empty((Tq, pf.Hq), dtype=torch.float32, device=dev),
            "gen_o": torch.empty((Tq, pf.Hq, pf.D), dtype=torch.bfloat16, device=dev),
            "gen_l": torch.empty((Tq, pf.Hq), dtype=torch.float32, device=dev),
            "dc_o": torch.empty((dc.B, dc.Hq, dc.D), dtype=torch.bfloat16, device=dev),
            "dc_l": torch.empty((dc.B, dc.Hq), dtype=torch.float32, device=dev),
            "d8_o": torch.empty((dc.B, dc.Hq, dc.D), dtype=torch.bfloat16, device=dev),
            "d8_l": torch.empty((dc.B, dc.Hq), dtype=torch.float32, device=dev),
        }

    def run(self):
        pf, dc, b = self.pf, self.dc, self.bufs
        pa.kv_page_write(pf.k_pool, pf.v_pool, pf.k_new, pf.v_new, pf.cu_new, pf.start_pos,
                         pf.block_tables)
        pa.paged_attn_prefill_varlen_splitk(
            pf.q, pf.k_pool, pf.v_pool, pf.cu_seqlens_q, pf.seq_lens_k, pf.block_tables,
            pf.scale, causal=True, max_q_len=pf.max_q_len, num_splits=self.pf_splits,
            out=b["pf_o"], lse=b["pf_l"], workspace=self.pf_ws)
        pa.paged_attn_prefill_varlen(
            pf.q, pf.k_pool, pf.v_pool, pf.cu_seqlens_q, pf.seq_lens_k, pf.block_tables,
            pf.scale, causal=True, max_q_len=pf.max_q_len, out=b["gen_o"], lse=b["gen_l"],
            window_left=1000, alibi_slopes=self.slopes)
        pa.kv_page_write(dc.k_pool, dc.v_pool, dc.k_new, dc.v_new, dc.cu_new, dc.start_pos,
                         dc.block_tables)
        pa.paged_attn_decode(dc.q, dc.k_pool, dc.v_pool, dc.block_tables, dc.seq_lens_k,
                             dc.scale, max_seq_len=8192, num_splits=self.dc_splits,
                             out=b["dc_o"], lse=b["dc_l"], workspace=self.dc_ws)
        pa.kv_page_write_fp8(self.kc, self.vc, dc.k_new, dc.v_new, dc.cu_new, dc.start_pos,
                             dc.block_tables, K_SCALE, V_SCALE)
        pa.paged_attn_decode_fp8(dc.q, self.kc, self.vc, dc.block_tables, dc.seq_lens_k,
                                 dc.scale, K_SCALE, V_SCALE, max_seq_len=8192,
                                 num_splits=self.dc_splits, out=b["d8_o"], lse=b["d8_l"],
                                 workspace=self.dc8_ws)

    def snapshot(self):
        snap = {}
        for k, t in self.bufs.items():
            snap[k] = bits(t).copy() if t.dtype == torch.bfloat16 else t.cpu().numpy().copy()
        for k, t in (("pf_kp", self.pf.k_pool), ("pf_vp", self.pf.v_pool),
                     ("dc_kp", self.dc.k_pool), ("dc_vp", self.dc.v_pool)):
            snap[k] = bits(t).copy()
        snap["kc"] = self.kc.cpu().numpy().copy()
        snap["vc"] = self.vc.cpu().numpy().copy()
        return snap

    def clear_outputs(self):
        for t in self.bufs.values():
            t.fill_(-7.0)


def _other_shapes(step):
    """Eager calls of other shapes on the same workspaces (their results are not kept)."""
    other = make_case("gother", hist_lens=[5000], q_lens=[700], write_new=True, causal=True,
                      Hq=8, Hkv=2, D=128, page_size=16, seed=74, device="cuda")
    pa.kv_page_write(other.k_pool, other.v_pool, other.k_new, other.v_new, other.cu_new,
                     other.start_pos, other.block_tables)
    pa.paged_attn_prefill_varlen_splitk(
        other.q, other.k_pool, other.v_pool, other.cu_seqlens_q, other.seq_lens_k,
        other.block_tables, other.scale, causal=True, max_q_len=other.max_q_len, num_splits=2,
        workspace=step.pf_ws)
    dc = step.dc
    pa.paged_attn_decode(dc.q[:2], dc.k_pool, dc.v_pool, dc.block_tables[:2],
                         dc.seq_lens_k[:2], dc.scale, max_seq_len=8192, num_splits=3,
                         workspace=step.dc_ws)
    pa.paged_attn_decode_fp8(dc.q[:3], step.kc, step.vc, dc.block_tables[:3],
                             dc.seq_lens_k[:3], dc.scale, K_SCALE, V_SCALE, max_seq_len=8192,
                             num_splits=2, workspace=step.dc8_ws)


def test_serving_step_graph_replays_match_eager(require_gpu):
    print("[graph] serving step: writes, split prefill, window+ALiBi prefill, bf16 and FP8 "
          "decode", flush=True)
    pf, dc = _cases()
    kp, vp = pools_after_write(pf)
    step = Step(pf, dc)
    step.run()
    torch.cuda.synchronize()
    ref = step.snapshot()

    # the eager step itself is the oracle's attention
    o_ref, l_ref = oracle_full(pf, kp, vp)
    assert_parity(as_f64(step.bufs["pf_o"]), o_ref, "graph step prefill")
    assert_lse(as_f64(step.bufs["pf_l"]), l_ref, "graph step prefill lse")

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step.run()
    torch.cuda.synchronize()
    for rep in range(4):
        step.clear_outputs()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = step.snapshot()
        for k in ref:
            assert np.array_equal(got[k], ref[k]), (rep, k)
        _other_shapes(step)
        torch.cuda.synchronize()


def test_prepared_calls_repeat_the_launches(require_gpu):
    """pa.prepared() replays a call's C launches with the arguments marshalled once:
    the replay reads the tensors' current contents (new queries written in place give
    the direct call's new result) and matches direct calls bit for bit."""
    print("[prepared] decode partials + reduce, prefill", flush=True)
    pf, dc = _cases()
    pa.kv_page_write(pf.k_pool, pf.v_pool, pf.k_new, pf.v_new, pf.cu_new, pf.start_pos,
                     pf.block_tables)
    pa.kv_page_write(dc.k_pool, dc.v_pool, dc.k_new, dc.v_new, dc.cu_new, dc.start_pos,
                     dc.block_tables)
    S = 3
    R = dc.B * dc.Hq
    po = torch.empty((R, S, dc.D), dtype=torch.float32, device="cuda")
    pl = torch.empty((R, S), dtype=torch.float32, device="cuda")
    out = torch.empty((R, dc.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((R,), dtype=torch.float32, device="cuda")
    pf_out = torch.empty((pf.q.shape[0], pf.Hq, pf.D), dtype=torch.bfloat16, device="cuda")

    def decode():
        pa.paged_attn_decode_partials(dc.q, dc.k_pool, dc.v_pool, dc.block_tables,
                                      dc.seq_lens_k, dc.scale, num_splits=S, max_seq_len=8192,
                                      partial_out=po, partial_lse=pl)
        pa.paged_attn_splitk_reduce(po, pl, out=out, lse=lse)

    def prefill():
        pa.paged_attn_prefill_varlen(pf.q, pf.k_pool, pf.v_pool, pf.cu_seqlens_q, pf.seq_lens_k,
                                     pf.block_tables, pf.scale, causal=True,
                                     max_q_len=pf.max_q_len, out=pf_out)

    run_d = pa.prepared(decode)
    run_p = pa.prepared(prefill)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda")
    for rep in range(3):
        if rep:
            gen.manual_seed(100 + rep)
            dc.q.copy_(torch.randn(dc.q.shape, generator=gen, device="cuda").to(torch.bfloat16))
            pf.q.copy_(torch.randn(pf.q.shape, generator=gen, device="cuda").to(torch.bfloat16))
        decode()
        prefill()
        torch.cuda.synchronize()
        ref = (bits(out).copy(), lse.cpu().numpy().copy(), bits(pf_out).copy())
        out.zero_()
        lse.zero_()
        pf_out.zero_()
        run_d()
        run_p()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), ref[0]), rep
        assert np.array_equal(lse.cpu().numpy(), ref[1]), rep
        assert np.array_equal(bits(pf_out), ref[2]), rep


def test_kernel_events_time_the_main_kernel(require_gpu):
    """kernel_events: the main kernel's dispatch stamps the pair; results are bitwise
    those of the call without events, and the stamped interval is positive and
    within the whole call's (split decode: partition kernel inside partition +
    merge; key-split prefill: prefill kernel inside prefill + merge)."""
    print("[events] decode, FP8 decode, prefill, split prefill", flush=True)
    pf, dc = _cases()
    step = Step(pf, dc)
    step.run()
    torch.cuda.synchronize()
    ref = step.snapshot()

    def ev_pair():
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        b.record()
        return a, b

    b = step.bufs
    calls = {
        "decode": lambda ev: pa.paged_attn_decode(
            dc.q, dc.k_pool, dc.v_pool, dc.block_tables, dc.seq_lens_k, dc.scale,
            max_seq_len=8192, num_splits=step.dc_splits, out=b["dc_o"], lse=b["dc_l"],
            workspace=step.dc_ws, kernel_events=ev),
        "decode_fp8": lambda ev: pa.paged_attn_decode_fp8(
            dc.q, step.kc, step.vc, dc.block_tables, dc.seq_lens_k, dc.scale, K_SCALE, V_SCALE,
            max_seq_len=8192, num_splits=step.dc_splits, out=b["d8_o"], lse=b["d8_l"],
            workspace=step.dc8_ws, kernel_events=ev),
        "prefill_split": lambda ev: pa.paged_attn_prefill_varlen_splitk(
            pf.q, pf.k_pool, pf.v_pool, pf.cu_seqlens_q, pf.seq_lens_k, pf.block_tables,
            pf.scale, causal=True, max_q_len=pf.max_q_len, num_splits=step.pf_splits,
            out=b["pf_o"], lse=b["pf_l"], workspace=step.pf_ws, kernel_events=ev),
        "prefill_general": lambda ev: pa.paged_attn_prefill_varlen(
            pf.q, pf.k_pool, pf.v_pool, pf.cu_seqlens_q, pf.seq_lens_k, pf.block_tables,
            pf.scale, causal=True, max_q_len=pf.max_q_len, out=b["gen_o"], lse=b["gen_l"],
            window_left=1000, alibi_slopes=step.slopes, kernel_events=ev),
    }
    torch.cuda.synchronize()
    for name, call in calls.items():
        kev = ev_pair()
        whole = ev_pair()
        torch.cuda.synchronize()
        step.clear_outputs()
        whole[0].record()
        call(kev)
        whole[1].record()
        torch.cuda.synchronize()
        k_ms, w_ms = kev[0].elapsed_time(kev[1]), whole[0].elapsed_time(whole[1])
        print(f"[events] {name}: kernel {k_ms * 1e3:.1f} us of {w_ms * 1e3:.1f} us", flush=True)
        assert 0.0 < k_ms <= w_ms, (name, k_ms, w_ms)
        got = step.snapshot()
        keys = {"decode": ("dc_o", "dc_l"), "decode_fp8": ("d8_o", "d8_l"),
                "prefill_split": ("pf_o", "pf_l"), "prefill_general": ("gen_o", "gen_l")}[name]
        for k in keys:
            assert np.array_equal(got[k], ref[k]), (name, k)
    with pytest.raises(ValueError):
        pa.paged_attn_decode(dc.q, dc.k_pool, dc.v_pool, dc.block_tables, dc.seq_lens_k,
                             dc.scale, max_seq_len=8192,
                             kernel_events=(torch.cuda.Event(enable_timing=True),
                                            torch.cuda.Event(enable_timing=True)))


def test_mixed_step_in_one_launch_graph_replays_match_eager(require_gpu):
    """The page write and the one-launch mixed step (paged_attn_mixed: key-split prefill
    chunks and decode rows in one kernel, then both merges) captured in a graph:
    every replay, with eager mixed calls of other shapes on the same workspace in
    between, gives the eager results bit for bit, and those match the oracle."""
    print("[graph] one-launch mixed step", flush=True)
    case = make_case("gmx", hist_lens=[2000, 0, 300, 4000, 17], q_lens=[512, 700, 1, 1, 1],
                     write_new=True, causal=True, Hq=8, Hkv=2, D=128, page_size=16, seed=80,
                     device="cuda")
    kp, vp = pools_after_write(case)
    t_pf = int(case.cu_seqlens_q[2])
    pf = (case.q[:t_pf].contiguous(), case.cu_seqlens_q[:3].contiguous(),
          case.seq_lens_k[:2].contiguous(), case.block_tables[:2].contiguous())
    dc = (case.q[t_pf:].contiguous(), case.block_tables[2:].contiguous(),
          case.seq_lens_k[2:].contiguous())
    need = pa.mixed_workspace_bytes(8, 2, 128, (2, t_pf, 700, 3), (3, 4001, 0))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    bufs = {"pf_o": torch.empty((t_pf, 8, 128), dtype=torch.bfloat16, device="cuda"),
            "pf_l": torch.empty((t_pf, 8), dtype=torch.float32, device="cuda"),
            "dc_o": torch.empty((3, 8, 128), dtype=torch.bfloat16, device="cuda"),
            "dc_l": torch.empty((3, 8), dtype=torch.float32, device="cuda")}

    def run():
        pa.kv_page_write(case.k_pool, case.v_pool, case.k_new, case.v_new, case.cu_new,
                         case.start_pos, case.block_tables)
        pa.paged_attn_mixed(case.k_pool, case.v_pool, case.scale, prefill=pf, decode=dc,
                            prefill_max_q_len=700, prefill_num_splits=3,
                            decode_max_seq_len=4001, decode_num_splits=0,
                            prefill_out=bufs["pf_o"], decode_out=bufs["dc_o"],
                            prefill_lse=bufs["pf_l"], decode_lse=bufs["dc_l"], workspace=ws)

    def snapshot():
        return {k: (bits(t).copy() if t.dtype == torch.bfloat16 else t.cpu().numpy().copy())
                for k, t in bufs.items()}

    run()
    torch.cuda.synchronize()
    ref = snapshot()
    o_ref, l_ref = oracle_full(case, kp, vp)
    assert_parity(as_f64(bufs["pf_o"]), o_ref[:t_pf], "graph mixed prefill")
    assert_parity(as_f64(bufs["dc_o"]), o_ref[t_pf:], "graph mixed decode")
    assert_lse(as_f64(bufs["dc_l"]), l_ref[t_pf:], "graph mixed decode lse")

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in bufs.values():
            t.fill_(-7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k in ref:
            assert np.array_equal(got[k], ref[k]), (rep, k)
        # other shapes on the same workspace: the first prefill chunk alone with 2 parts,
        # two decode rows with 7 splits
        pa.paged_attn_mixed(case.k_pool, case.v_pool, case.scale,
                            prefill=(pf[0][:512], pf[1][:2], pf[2][:1], pf[3][:1]),
                            decode=(dc[0][:2], dc[1][:2], dc[2][:2]), prefill_num_splits=2,
                            decode_num_splits=7, workspace=ws)
        torch.cuda.synchronize()


def test_prepared_mixed_step_repeats_the_launch(require_gpu):
    """pa.prepared() around the one-launch mixed step (its structs marshalled once, the
    workspace the binding allocated held by the returned function): replays after new
    queries are written in place match direct calls bit for bit."""
    print("[prepared] one-launch mixed step", flush=True)
    case = make_case("pmx", hist_lens=[1500, 0, 200, 3000], q_lens=[512, 600, 1, 1],
                     write_new=True, causal=True, Hq=8, Hkv=2, D=128, page_size=16, seed=90,
                     device="cuda")
    pa.kv_page_write(case.k_pool, case.v_pool, case.k_new, case.v_new, case.cu_new,
                     case.start_pos, case.block_tables)
    t_pf = int(case.cu_seqlens_q[2])
    q_pf = case.q[:t_pf].contiguous()
    q_d = case.q[t_pf:].contiguous()
    pf = (q_pf, case.cu_seqlens_q[:3].contiguous(), case.seq_lens_k[:2].contiguous(),
          case.block_tables[:2].contiguous())
    dc = (q_d, case.block_tables[2:].contiguous(), case.seq_lens_k[2:].contiguous())
    o_p = torch.empty((t_pf, 8, 128), dtype=torch.bfloat16, device="cuda")
    o_d = torch.empty((2, 8, 128), dtype=torch.bfloat16, device="cuda")

    def step():
        pa.paged_attn_mixed(case.k_pool, case.v_pool, case.scale, prefill=pf, decode=dc,
                            prefill_max_q_len=600, prefill_num_splits=2,
                            decode_max_seq_len=3001, prefill_out=o_p, decode_out=o_d)

    run = pa.prepared(step)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda")
    for rep in range(3):
        if rep:
            gen.manual_seed(200 + rep)
            q_pf.copy_(torch.randn(q_pf.shape, generator=gen, device="cuda").to(torch.bfloat16))
            q_d.copy_(torch.randn(q_d.shape, generator=gen, device="cuda").to(torch.bfloat16))
        step()
        torch.cuda.synchronize()
        ref = (bits(o_p).copy(), bits(o_d).copy())
        o_p.zero_()
        o_d.zero_()
        run()
        torch.cuda.synchronize()
        assert np.array_equal(bits(o_p), ref[0]), rep
        assert np.array_equal(bits(o_d), ref[1]), rep
