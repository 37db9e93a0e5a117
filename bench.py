"""Benchmark of the paged-KV attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Headline: Qwen2.5-7B-shaped one-layer decode (batch 32, context 8192, Hq 28,
Hkv 4, D 128, page size 16) -- the paged split-K decode plus its merge, inputs
resident in HBM.  Value = algorithmic KV-read GB/s (every attended K and V
element once per KV head, plus Q, O, used table entries and lengths).  Several
copies of the pools are rotated so that no step finds its KV in the 256 MiB
last-level cache.  Secondary lines (same JSON object): the same decode over
FP8 E4M3 pools (bytes counted at one per K/V element), dense causal prefill
TFLOP/s (4 x 4096, Hq 32, Hkv 8), long-context decode (8 x 131072), a 512-token
prefill chunk over a 32,768-token history (key-split prefill), and the mixed
ragged step, each timed the same way.

For the HBM-bound headline the roofline object also carries the bandwidth of a
plain streaming read of a 4 GiB buffer measured on the same GPU (libpa_stream.so)
and the dominant kernel's fraction of it.

One JSON line is printed.  Only one GPU is used: --gpus above 1 is refused.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "decode KV-read GB/s (% HBM peak); causal prefill TFLOP/s (% MFMA peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--settle-ms", type=float, default=0.0,
                   help="after the warm-up steps, run untimed steps for this many more "
                        "milliseconds before timing the headline workload (the secondary "
                        "figures always take %g ms)" % SECONDARY_SETTLE_MS)
    p.add_argument("--workload", default="qwen7b_decode",
                   choices=["qwen7b_decode", "qwen7b_decode_fp8", "long_history_chunk",
                            "long_decode", "long_decode_auto", "causal_prefill",
                            "causal_prefill_fp8", "causal_prefill_block_map",
                            "mixed_ragged", "mixed_ragged_two_streams", "tiny_decode",
                            "qwen7b_decode_warm"])
    p.add_argument("--num-splits", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--traffic-pass", action="store_true",
                   help="run only a 1 GiB device copy and a few launches of the workload's "
                        "dominant kernel, for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE "
                        "collection (workloads: " + ", ".join(sorted(TRAFFIC)) + ")")
    p.add_argument("--record-traffic", metavar="DIR",
                   help="no GPU work: read the counter CSVs of the two --traffic-pass runs "
                        "of --workload under DIR/pmc_<workload>_FETCH_SIZE and "
                        "DIR/pmc_<workload>_WRITE_SIZE and write the workload's traffic "
                        "record under profiles/")
    return p.parse_args()


# ---------------------------------------------------------------------------
# steps
# ---------------------------------------------------------------------------

class DecodeStep:
    """One paged_attn_decode of the whole batch over one of `copies` rotated pool copies
    (with several partitions: the partition kernel, then the split-K merge)."""

    def __init__(self, name, copies, num_splits=0):
        import torch
        import paged_kv_flashattention_amd as pa
        from workloads import make_config, units
        self.pa = pa
        self.case = make_config(name, "cuda")
        c = self.case
        self.kv = [(c.k_pool, c.v_pool)]
        for i in range(1, copies):
            self.kv.append((c.k_pool.clone(), c.v_pool.clone()))
        self.S = num_splits if num_splits > 0 else pa.decode_num_splits(c.B, c.Hkv,
                                                                        c.max_seq_len)
        self.out = torch.empty((c.B, c.Hq, c.D), dtype=torch.bfloat16, device="cuda")
        need = pa.decode_workspace_bytes(c.B, c.Hq, c.Hkv, c.D, c.max_seq_len, self.S)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        self.po = torch.empty((c.B * c.Hq, self.S, c.D), dtype=torch.float32, device="cuda")
        self.pl = torch.empty((c.B * c.Hq, self.S), dtype=torch.float32, device="cuda")
        self.i = 0
        self.units = units.decode_bytes(c.seq_lens, c.Hq, c.Hkv, c.D, c.page_size)
        self.unit_name = "GB/s"

    def __call__(self):
        c = self.case
        kp, vp = self.kv[self.i % len(self.kv)]
        self.i += 1
        self.pa.paged_attn_decode(c.q, kp, vp, c.block_tables, c.seq_lens_k, c.scale,
                                  max_seq_len=c.max_seq_len, num_splits=self.S, out=self.out,
                                  workspace=self.ws, kernel_events=next_events(self))

    def partials(self):
        c = self.case
        kp, vp = self.kv[self.i % len(self.kv)]
        self.i += 1
        self.pa.paged_attn_decode_partials(c.q, kp, vp, c.block_tables, c.seq_lens_k, c.scale,
                                           num_splits=self.S, max_seq_len=c.max_seq_len,
                                           partial_out=self.po, partial_lse=self.pl)

    def partition_launches(self, launches):
        """`launches` back-to-back partition-kernel launches over the rotated pool
        copies (what the counter runs profile)."""
        for _ in range(launches):
            self.partials()

    def config(self):
        c = self.case
        return {"workload": c.name, "batch": c.B, "context": c.max_seq_len, "Hq": c.Hq,
                "Hkv": c.Hkv, "head_dim": c.D, "page_size": c.page_size,
                "num_splits": self.S, "pool_copies_rotated": len(self.kv)}


class Fp8DecodeStep(DecodeStep):
    """The same decode over FP8 E4M3 pools: seeded random codes of the same shape
    (one byte per element), per-pool scales, rotated copies as above."""

    K_SCALE, V_SCALE = 0.02, 0.05

    def __init__(self, name, copies, num_splits=0):
        super().__init__(name, 1, num_splits)
        from workloads import random_e4m3_codes, units
        c = self.case
        shape = tuple(c.k_pool.shape)
        c.k_pool = c.v_pool = None
        self.kv = [(random_e4m3_codes(shape, 8000 + 2 * i, "cuda"),
                    random_e4m3_codes(shape, 8001 + 2 * i, "cuda")) for i in range(copies)]
        self.units = units.decode_bytes(c.seq_lens, c.Hq, c.Hkv, c.D, c.page_size,
                                        kv_elem_bytes=1)

    def __call__(self):
        c = self.case
        kp, vp = self.kv[self.i % len(self.kv)]
        self.i += 1
        self.pa.paged_attn_decode_fp8(c.q, kp, vp, c.block_tables, c.seq_lens_k, c.scale,
                                      self.K_SCALE, self.V_SCALE, max_seq_len=c.max_seq_len,
                                      num_splits=self.S, out=self.out, workspace=self.ws,
                                      kernel_events=next_events(self))

    def config(self):
        return dict(super().config(), kv_format="fp8-e4m3")


class PrefillStep:
    """kv_page_write is done once at setup; each step is one prefill_varlen call (with
    `splitk`, one prefill_varlen_splitk call with the key-part count that
    paged_attn_prefill_plan_splits gives for the lengths: the prefill kernel, then the
    merge of the split tiles).  Steps rotate over `copies` copies of Q, the pools and
    the output, so that a step does not find its inputs in the 256 MiB last-level
    cache (two copies of the causal prefill's Q, K, V and O are 664 MB)."""

    def __init__(self, name, splitk=False, copies=2):
        import torch
        import paged_kv_flashattention_amd as pa
        from workloads import make_config, units
        self.pa = pa
        self.case = c = make_config(name, "cuda")
        pa.kv_page_write(c.k_pool, c.v_pool, c.k_new, c.v_new, c.cu_new, c.start_pos,
                         c.block_tables)
        self.out = torch.empty((c.T, c.Hq, c.D), dtype=torch.bfloat16, device="cuda")
        self.units = units.prefill_flops(c.seq_lens, c.q_lens, c.Hq, c.D, c.causal)
        self.unit_name = "TFLOP/s"
        # key parts planned from the host lengths, as a scheduler would
        self.S = pa.prefill_plan_splits(c.q_lens, c.seq_lens, c.Hq) if splitk else 1
        need = pa.prefill_workspace_bytes(c.B, c.T, c.max_q_len, c.Hq, c.D, self.S)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        self.splitk = splitk
        self.sets = [(c.q, c.k_pool, c.v_pool, self.out)]
        for _ in range(1, copies):
            self.sets.append((c.q.clone(), c.k_pool.clone(), c.v_pool.clone(),
                              torch.empty_like(self.out)))
        self.i = 0

    def __call__(self):
        c = self.case
        q, kp, vp, out = self.sets[self.i % len(self.sets)]
        self.i += 1
        if self.splitk:
            self.pa.paged_attn_prefill_varlen_splitk(
                q, kp, vp, c.cu_seqlens_q, c.seq_lens_k, c.block_tables, c.scale,
                causal=True, max_q_len=c.max_q_len, num_splits=self.S, out=out,
                workspace=self.ws, kernel_events=next_events(self))
            return
        self.pa.paged_attn_prefill_varlen(q, kp, vp, c.cu_seqlens_q, c.seq_lens_k,
                                          c.block_tables, c.scale, causal=True,
                                          max_q_len=c.max_q_len, out=out,
                                          kernel_events=next_events(self))

    def config(self):
        c = self.case
        cfg = {"workload": c.name, "batch": c.B, "q_len": c.max_q_len, "Hq": c.Hq,
               "Hkv": c.Hkv, "head_dim": c.D, "page_size": c.page_size, "causal": True,
               "input_copies_rotated": len(self.sets)}
        if self.splitk:
            cfg.update(history=max(c.seq_lens) - c.max_q_len, key_parts=self.S)
        return cfg


class BlockMapPrefillStep(PrefillStep):
    """The causal prefill with a block map on top (64 x 64 blocks): every query block
    sees the 4 key blocks up to its own and every 8th block before them (23 % of the
    causal pairs).  The rate counts the pairs the map leaves visible."""

    def __init__(self, name):
        import numpy as np
        import torch
        from workloads import local_strided_block_map, units
        super().__init__(name)
        c = self.case
        qb, kb = -(-c.max_q_len // 64), -(-max(c.seq_lens) // 64)
        bm = np.stack([local_strided_block_map(qb, kb)] * c.B)
        self.bm = torch.from_numpy(bm).cuda()
        self.units = 4 * c.D * c.Hq * units.block_map_pairs(c.seq_lens, c.q_lens, True, bm)

    def __call__(self):
        c = self.case
        q, kp, vp, out = self.sets[self.i % len(self.sets)]
        self.i += 1
        self.pa.paged_attn_prefill_varlen(q, kp, vp, c.cu_seqlens_q, c.seq_lens_k,
                                          c.block_tables, c.scale, causal=True,
                                          max_q_len=c.max_q_len, out=out, block_map=self.bm,
                                          kernel_events=next_events(self))

    def config(self):
        cfg = super().config()
        cfg["block_map"] = "local 4 + every 8th of 64 x 64 blocks"
        return cfg


class Fp8PrefillStep(PrefillStep):
    """The same causal prefill over FP8 E4M3 pools: seeded random codes of the
    pools' shape with per-pool scales (the queries stay bf16)."""

    K_SCALE, V_SCALE = 0.02, 0.05

    def __init__(self, name, copies=2):
        super().__init__(name, copies=1)
        import torch
        from workloads import random_e4m3_codes
        c = self.case
        shape = tuple(c.k_pool.shape)
        c.k_pool = c.v_pool = None
        self.sets = [(c.q if i == 0 else c.q.clone(),
                      random_e4m3_codes(shape, 8100 + 2 * i, "cuda"),
                      random_e4m3_codes(shape, 8101 + 2 * i, "cuda"),
                      self.out if i == 0 else torch.empty_like(self.out))
                     for i in range(copies)]

    def __call__(self):
        c = self.case
        q, kc, vc, out = self.sets[self.i % len(self.sets)]
        self.i += 1
        self.pa.paged_attn_prefill_varlen_fp8(
            q, kc, vc, c.cu_seqlens_q, c.seq_lens_k, c.block_tables, c.scale,
            self.K_SCALE, self.V_SCALE, causal=True, max_q_len=c.max_q_len, out=out,
            kernel_events=next_events(self))

    def config(self):
        return dict(super().config(), kv_format="fp8-e4m3")


class MixedStep:
    """The mixed ragged step: write 2,578 new tokens, prefill the 5 chunks, decode 18 rows.

    The prefill's key-part count comes from paged_attn_prefill_plan_splits over the
    chunks' host lengths (as a scheduler would plan it), the decode's split count
    from the library's rule.  With one_launch (the workload's figure) the prefill and
    the decode run in one kernel (paged_attn_mixed) after the write, then the two
    merges, all on the launch stream.  Without it the prefill chunks and the decode
    rows, which read disjoint outputs and only read the pools after the write, run as
    separate kernels: the decode on a second stream (default priority) after the
    write, issued behind the prefill so that its work-groups fill the slots the
    prefill leaves; the step ends when both have finished (the launch stream waits for
    the second one)."""

    def __init__(self, name="mixed_ragged", one_launch=True):
        import torch
        import paged_kv_flashattention_amd as pa
        from workloads import make_config, units
        self.pa = pa
        self.one_launch = one_launch
        self.case = c = make_config(name, "cuda")
        n = 5
        self.t_pf = int(c.cu_seqlens_q[n])
        self.cu_pf = c.cu_seqlens_q[:n + 1].contiguous()
        self.lens_pf = c.seq_lens_k[:n].contiguous()
        self.bt_pf = c.block_tables[:n].contiguous()
        self.q_pf = c.q[:self.t_pf].contiguous()
        self.q_d = c.q[self.t_pf:].contiguous()
        self.lens_d = c.seq_lens_k[n:].contiguous()
        self.bt_d = c.block_tables[n:].contiguous()
        self.max_d = max(c.seq_lens[n:])
        self.max_q = max(c.q_lens[:n])
        self.S_pf = pa.prefill_plan_splits(c.q_lens[:n], c.seq_lens[:n], c.Hq, causal=True)
        need = pa.prefill_workspace_bytes(n, self.t_pf, self.max_q, c.Hq, c.D, self.S_pf)
        self.ws_pf = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        self.S = pa.decode_num_splits(c.B - n, c.Hkv, self.max_d)
        need = pa.decode_workspace_bytes(c.B - n, c.Hq, c.Hkv, c.D, self.max_d, self.S)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        self.out_pf = torch.empty((self.t_pf, c.Hq, c.D), dtype=torch.bfloat16, device="cuda")
        self.out_d = torch.empty((c.B - n, c.Hq, c.D), dtype=torch.bfloat16, device="cuda")
        self.flops = units.prefill_flops(c.seq_lens[:n], c.q_lens[:n], c.Hq, c.D, True)
        self.bytes = units.decode_bytes(c.seq_lens[n:], c.Hq, c.Hkv, c.D, c.page_size)
        self.units = self.flops
        self.unit_name = "TFLOP/s"
        self.side = torch.cuda.Stream()
        if one_launch:
            # one kernel for both parts (paged_attn_mixed) with the same key parts and
            # the library's decode split count for that launch, then the two merges,
            # all on the launch stream
            need = pa.mixed_workspace_bytes(c.Hq, c.Hkv, c.D, (n, self.t_pf, self.max_q, self.S_pf),
                                            (c.B - n, self.max_d, 0))
            self.ws_mixed = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
            self.launch = None

    def __call__(self):
        import torch
        c = self.case
        pa = self.pa
        main = torch.cuda.current_stream()
        pa.kv_page_write(c.k_pool, c.v_pool, c.k_new, c.v_new, c.cu_new, c.start_pos,
                         c.block_tables)
        if self.one_launch:
            pa.paged_attn_mixed(c.k_pool, c.v_pool, c.scale,
                                prefill=(self.q_pf, self.cu_pf, self.lens_pf, self.bt_pf),
                                decode=(self.q_d, self.bt_d, self.lens_d),
                                prefill_max_q_len=self.max_q, prefill_num_splits=self.S_pf,
                                decode_max_seq_len=self.max_d, decode_num_splits=0,
                                prefill_out=self.out_pf, decode_out=self.out_d,
                                workspace=self.ws_mixed)
            if self.launch is None:
                self.launch = pa.describe_launch()
            return
        self.side.wait_stream(main)
        pa.paged_attn_prefill_varlen_splitk(self.q_pf, c.k_pool, c.v_pool, self.cu_pf,
                                            self.lens_pf, self.bt_pf, c.scale, causal=True,
                                            max_q_len=self.max_q, num_splits=self.S_pf,
                                            out=self.out_pf, workspace=self.ws_pf)
        with torch.cuda.stream(self.side):
            pa.paged_attn_decode(self.q_d, c.k_pool, c.v_pool, self.bt_d, self.lens_d, c.scale,
                                 max_seq_len=self.max_d, num_splits=self.S, out=self.out_d,
                                 workspace=self.ws)
        main.wait_stream(self.side)

    def config(self):
        c = self.case
        cfg = {"workload": c.name, "requests": c.B, "prefill_chunks": 5, "chunk_len": 512,
               "decode_rows": c.B - 5, "Hq": c.Hq, "Hkv": c.Hkv, "head_dim": c.D,
               "page_size": c.page_size, "prefill_key_parts": self.S_pf,
               "decode_splits": self.S, "launch": "prefill and decode kernels on two streams"}
        if self.one_launch:
            import re
            m = re.search(r"x (\d+) splits", self.launch or "")
            cfg.update(decode_splits=int(m.group(1)) if m else None,
                       launch="one kernel for both parts (paged_attn_mixed)")
        return cfg


class GraphStep:
    """`calls` consecutive calls of a step captured in one HIP graph
    (torch.cuda.CUDAGraph around the library's launches on the capture stream, the
    mixed step's second stream forked from and joined back into it); one replay is
    one timed call doing `calls` steps' work.  Every call in these steps is
    capturable as it stands: no memset, no allocation, no host synchronisation
    (tests/test_graphs.py replays such a step and checks every replay bit for bit
    against the eager calls)."""

    def __init__(self, inner, calls):
        import torch
        self.inner = inner
        self.calls = calls
        self.units = inner.units * calls
        self.unit_name = inner.unit_name
        for _ in range(2):                      # eager first: one-time library set-up
            inner()
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for _ in range(calls):
                inner()
        torch.cuda.synchronize()

    def __call__(self):
        self.graph.replay()

    def config(self):
        return dict(self.inner.config(), hip_graph=f"{self.calls} calls per replay")


def make_step(name, num_splits=0):
    if name == "qwen7b_decode_fp8":
        return Fp8DecodeStep("qwen7b_decode", copies=3, num_splits=num_splits)
    if name == "qwen7b_decode":
        return DecodeStep(name, copies=3, num_splits=num_splits)
    if name == "qwen7b_decode_warm":
        # one pool copy: the same 537 MB every step, so whatever of it the 256 MiB
        # last-level cache keeps between steps is read from there (the warm figure)
        return DecodeStep("qwen7b_decode", copies=1, num_splits=num_splits)
    if name == "long_decode":
        # the workload is stated with 64 partitions; --num-splits overrides
        return DecodeStep(name, copies=1, num_splits=num_splits or 64)
    if name == "long_decode_auto":
        # the same decode with the library's own split count
        return DecodeStep("long_decode", copies=1, num_splits=num_splits)
    if name == "tiny_decode":
        return DecodeStep(name, copies=1, num_splits=num_splits)
    if name == "causal_prefill":
        return PrefillStep(name)
    if name == "causal_prefill_fp8":
        return Fp8PrefillStep("causal_prefill")
    if name == "causal_prefill_block_map":
        return BlockMapPrefillStep("causal_prefill")
    if name == "long_history_chunk":
        return PrefillStep(name, splitk=True)
    if name == "mixed_ragged_two_streams":
        return MixedStep("mixed_ragged", one_launch=False)
    return MixedStep(name, one_launch=True)


def next_events(step):
    """The kernel-event pair for this call of a timed step, or None outside timing."""
    it = getattr(step, "events", None)
    return next(it) if it is not None else None


# Untimed running before the secondary figures are timed.  A GPU that has been idle
# runs a heavy kernel at full speed for its first 1-2 ms of sustained load, then
# 15-25 % slower for several milliseconds, and only after 10-30 ms back at a steady
# rate (kernel traces of the causal prefill: 580 us, then 730 us, then 575 us per
# launch).  Five warm-up steps of a 0.6 ms kernel end inside that dip, so the
# secondary figures first run their own steps untimed for this long.
SECONDARY_SETTLE_MS = 50.0


def time_step(step, steps, warmup, kernel_events=True, settle_ms=0.0):
    """Warm up, then time exactly `steps` calls bracketed by synchronisations.

    After the `warmup` calls, more untimed calls run until `settle_ms` milliseconds
    of wall time have passed (0: none), so that the timed calls find the engine at
    its sustained clock.

    Returns (wall ms per step, event ms per step, dominant-kernel ms or None).  The
    step's time comes from HIP events recorded on the launch stream (torch's current
    stream) before the first and after the last call, with nothing else in the
    stream.  Then the same `steps` calls run once more, each handing its main
    kernel's dispatch a pair of events that the dispatch itself stamps with that
    kernel's start and end (the library's kernel_events option): their average is
    the dominant kernel's duration.  Stamped dispatches lengthen a step by a few
    microseconds on this runtime, which is why the timed pass carries none."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    step.settle_calls = 0
    if settle_ms > 0:
        t_end = time.perf_counter() + settle_ms * 1e-3
        while time.perf_counter() < t_end:
            for _ in range(8):
                step()
            step.settle_calls += 8
            torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ev = start.elapsed_time(stop) / steps
    if not kernel_events or isinstance(step, (MixedStep, GraphStep, PreparedStep)):
        return wall, ev, None
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    for a, b in pairs:                         # HIP events are created when first recorded
        a.record()
        b.record()
    torch.cuda.synchronize()
    step.events = iter(pairs)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    step.events = None
    durs = sorted(a.elapsed_time(b) for a, b in pairs)
    step.kernel_ms_median = durs[len(durs) // 2]
    step.kernel_ms_min = durs[0]
    return wall, ev, sum(durs) / steps


def rate(units, ms, unit_name):
    if unit_name == "GB/s":
        return units / (ms * 1e-3) / 1e9
    return units / (ms * 1e-3) / 1e12


# ---------------------------------------------------------------------------
# HBM traffic of the dominant kernel, from rocprofv3 counters
# ---------------------------------------------------------------------------

# per workload: the recorded counter figures of its dominant kernel, the sources that
# kernel is built from, and the kernel's name as the profiler reports it (a prefix)
_DECODE_SRC = ["decode.hip", "decode_item.hpp", "decode_walk.inc", "common.hpp", "kernels.hpp"]
_PREFILL_SRC = ["prefill.hip", "decode_item.hpp", "decode_walk.inc", "common.hpp",
                "kernels.hpp"]
TRAFFIC = {
    "qwen7b_decode": ("decode_partition_qwen7b_decode_traffic.json", _DECODE_SRC,
                      "pa::decode_partition_kernel<"),
    "long_decode": ("decode_group_long_decode_traffic.json", _DECODE_SRC,
                    "pa::decode_group_kernel<"),
    "long_decode_auto": ("decode_partition_long_decode_auto_traffic.json", _DECODE_SRC,
                         "pa::decode_partition_kernel<"),
    "causal_prefill": ("prefill_causal_prefill_traffic.json", _PREFILL_SRC,
                       "pa::prefill_kernel<"),
    "long_history_chunk": ("prefill_long_history_chunk_traffic.json", _PREFILL_SRC,
                           "pa::prefill_kernel<"),
}
COPY_BYTES = 1 << 30           # the calibration copy reads and writes this many bytes


def source_digest(workload):
    """sha256 over the sources the workload's dominant kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "paged_kv_flashattention_amd", "csrc")
    for f in TRAFFIC[workload][1]:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """Bytes per launch of the workload's dominant kernel (FETCH_SIZE + WRITE_SIZE,
    each scaled by the same counter's reading for a copy of known size), as recorded
    from the counter runs -- or None when there is no record or the kernel's sources
    changed since."""
    if workload not in TRAFFIC:
        return None
    try:
        with open(os.path.join(ROOT, "profiles", TRAFFIC[workload][0])) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest(workload):
        return None
    return rec.get("bytes_per_launch")


def traffic_pass(steps, workload):
    """What the counter runs profile: a plain device copy of COPY_BYTES (the
    calibration), then `steps` launches of the workload's dominant kernel as the
    timed steps launch them (decode: the partition kernel over the rotated pool
    copies; prefill: whole steps, whose only kernel is the prefill kernel)."""
    import torch
    if workload not in TRAFFIC:
        raise SystemExit(f"--traffic-pass covers {sorted(TRAFFIC)}, not {workload}")
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    step = make_step(workload, 0)
    if isinstance(step, DecodeStep):
        step.partition_launches(steps)
    else:
        for _ in range(steps):
            step()
    torch.cuda.synchronize()
    log(f"[bench] traffic pass: copy of {COPY_BYTES} bytes, {steps} {workload} launches; "
        f"sources {source_digest(workload)[:16]}")


def record_traffic(workload, pmc_dir):
    """The traffic record of `workload` from the counter CSVs of its two traffic-pass
    runs (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).  Each
    counter is scaled by its own reading for the pass's calibration copy of
    COPY_BYTES (read once, written once), and the dominant kernel's dispatches are
    averaged: bytes per launch = (FETCH_SIZE x fetch scale + WRITE_SIZE x write
    scale) x 1024.  Written to profiles/ with the digest of the kernel's sources."""
    import csv
    from workloads import config_shape, units
    fname, _, kname = TRAFFIC[workload]

    def per_dispatch(counter):
        path = os.path.join(pmc_dir, f"pmc_{workload}_{counter}", "run_counter_collection.csv")
        agg = {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                k = (int(r["Dispatch_Id"]), name[5:] if name.startswith("void ") else name)
                agg[k] = agg.get(k, 0.0) + float(r["Counter_Value"])
        return agg

    f, w = per_dispatch("FETCH_SIZE"), per_dispatch("WRITE_SIZE")
    kib = COPY_BYTES / 1024
    # the calibration copy: the one large copyBuffer dispatch
    cf = max(v for (_, n), v in f.items() if "copyBuffer" in n)
    cw = max(v for (_, n), v in w.items() if "copyBuffer" in n)
    fs, ws = kib / cf, kib / cw
    kf = [v for (_, n), v in sorted(f.items()) if n.startswith(kname)]
    kw = [v for (_, n), v in sorted(w.items()) if n.startswith(kname)]
    names = sorted({n for (_, n) in f if n.startswith(kname)})
    fk, wk = sum(kf) / len(kf), sum(kw) / len(kw)
    rec = {"kernel": names[0] if len(names) == 1 else names, "workload": workload,
           "fetch_kib_per_launch": round(fk, 3), "fetch_kib_range": [min(kf), max(kf)],
           "write_kib_per_launch": round(wk, 3), "write_kib_range": [min(kw), max(kw)],
           "launches": len(kf),
           "calibration": {"copy_bytes": COPY_BYTES, "fetch_kib": cf, "write_kib": cw,
                           "fetch_scale": round(fs, 6), "write_scale": round(ws, 6)},
           "bytes_per_launch": int(round((fk * fs + wk * ws) * 1024))}
    c = config_shape("long_decode" if workload == "long_decode_auto" else workload)
    if workload in ("causal_prefill", "long_history_chunk"):
        rec["minimum_bytes_per_launch"] = units.prefill_bytes(c["seq_lens"], c["q_lens"],
                                                              c["Hq"], c["Hkv"], c["D"])
        rec["minimum_bytes_note"] = ("Q and O once, K and V once per KV head; the kernel is "
                                     "bound by its matrix work, not by these bytes")
    else:
        rec["algorithmic_bytes_per_launch"] = units.decode_bytes(
            c["seq_lens"], c["Hq"], c["Hkv"], c["D"], c["page_size"])
    rec["source_sha256"] = source_digest(workload)
    rec["commands"] = [
        f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL 150 rocprofv3 --pmc {k} "
        f"--output-format csv -d $OUT/pmc_{workload}_{k} -o run -- python3 "
        f"$REPO/bench.py --traffic-pass --workload {workload} --steps 6"
        for k in ("FETCH_SIZE", "WRITE_SIZE")] + [
        f"python3 bench.py --workload {workload} --record-traffic $OUT"]
    with open(os.path.join(ROOT, "profiles", fname), "w") as fh:
        json.dump(rec, fh, indent=1)
    log(f"[bench] {workload}: {rec['bytes_per_launch']} bytes per launch -> profiles/{fname}")


# ---------------------------------------------------------------------------
# the box's streaming-read bandwidth (reference for the HBM-bound kernels)
# ---------------------------------------------------------------------------

STREAM_BYTES = 4 << 30


def stream_read_gbs(iters=10):
    """Best GB/s of a plain streaming read of a 4 GiB buffer (libpa_stream.so, built
    with the library: each work-group streams one contiguous chunk), over a few grid
    sizes; HIP events on the launch stream."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "paged_kv_flashattention_amd", "libpa_stream.so")
    lib = ctypes.CDLL(path)
    fn = lib.pa_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                   ctypes.c_void_p]
    buf = torch.empty(STREAM_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    best = (0.0, 0)
    for blocks in (1024, 4096, 16384, 65536, 262144):
        sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
        s = torch.cuda.current_stream().cuda_stream
        for _ in range(2):
            if fn(buf.data_ptr(), STREAM_BYTES, sink.data_ptr(), blocks, s):
                raise RuntimeError("pa_stream_read rejected its arguments")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(iters):
            fn(buf.data_ptr(), STREAM_BYTES, sink.data_ptr(), blocks, s)
        b.record()
        torch.cuda.synchronize()
        gbs = STREAM_BYTES / (a.elapsed_time(b) / iters * 1e-3) / 1e9
        best = max(best, (gbs, blocks))
    del buf
    torch.cuda.empty_cache()
    return best


# ---------------------------------------------------------------------------
# oracle baseline on the host cores
# ---------------------------------------------------------------------------

def host_cores():
    """(cores this process may run on, BLAS threads the oracle's NumPy uses)."""
    cores = len(os.sched_getaffinity(0))
    try:
        # the oracle's NumPy runs single-threaded except inside BLAS calls
        from threadpoolctl import threadpool_info
        blas = max([1] + [int(p.get("num_threads", 1)) for p in threadpool_info()])
    except Exception:
        blas = None
    return cores, blas


def cpu_baseline(step, min_s=10.0, budget_s=15.0):
    """The float64 oracle, as it stands, on a bounded sample of the same workload.

    Decode: passes over the batch's sequences (each sequence's pages copied to the
    host once, untimed) until at least min_s seconds of oracle time, stopping at
    budget_s; algorithmic GB/s.  Causal prefill: whole (sequence, query head)
    planes -- every row of one head over its sequence's keys, the oracle given that
    sequence's pages and the KV head the query head reads -- until min_s; GFLOP/s
    of algorithmic prefill work."""
    if isinstance(step, PrefillStep) and not isinstance(step, (Fp8PrefillStep,
                                                               BlockMapPrefillStep)) \
            and not step.splitk:
        return cpu_baseline_prefill(step, min_s, budget_s)
    import numpy as np
    import oracle
    from workloads import bits, units
    cores, blas = host_cores()
    c = step.case
    if not isinstance(step, DecodeStep) or isinstance(step, Fp8DecodeStep):
        return None
    import torch
    bt = c.block_tables.cpu().numpy()
    lens = c.seq_lens_k.cpu().numpy()
    q = bits(c.q)
    host = []
    done, t_used, nbytes = 0, 0.0, 0
    while t_used < min_s:
        for b in range(c.B):
            if len(host) <= b:
                n_pages = -(-int(lens[b]) // c.page_size)
                pages = torch.as_tensor(bt[b, :n_pages].astype(np.int64), device="cuda")
                host.append((bits(c.k_pool[pages]), bits(c.v_pool[pages]),
                             np.arange(n_pages, dtype=np.int32)[None]))
            kp, vp, local_bt = host[b]
            t0 = time.perf_counter()
            oracle.attention_ref(q[b:b + 1], kp, vp, local_bt, lens[b:b + 1],
                                 np.array([0, 1]), c.scale, False, c.page_size)
            t_used += time.perf_counter() - t0
            nbytes += units.decode_bytes([int(lens[b])], c.Hq, c.Hkv, c.D, c.page_size)
            done += 1
            if t_used >= budget_s:
                break
        if t_used >= budget_s:
            break
    return {"value": nbytes / t_used / 1e9, "unit": "GB/s", "cores": cores,
            "blas_threads": blas, "kind": "oracle",
            "sample": f"{c.name}: {done} sequence decodes ({done / c.B:.1f} passes over the "
                      f"{c.B} sequences), all {c.Hq} query heads, float64 NumPy, "
                      f"{t_used:.1f} s of oracle time"}


def cpu_baseline_prefill(step, min_s=10.0, budget_s=15.0):
    import numpy as np
    import oracle
    from workloads import bits, units
    cores, blas = host_cores()
    c = step.case
    G = c.Hq // c.Hkv
    bt = c.block_tables.cpu().numpy()
    cu = c.cu_seqlens_q.cpu().numpy()
    lens = c.seq_lens
    q = bits(c.q)
    kp, vp = bits(c.k_pool), bits(c.v_pool)          # the pools after the step's write
    done, t_used, flops = 0, 0.0, 0
    planes = [(b, h) for h in range(c.Hq) for b in range(c.B)]
    for b, h in planes:
        L = int(lens[b])
        n = -(-L // c.page_size)
        pages = bt[b, :n].astype(np.int64)
        kvh = h // G
        kb = np.ascontiguousarray(kp[pages][:, :, kvh:kvh + 1])
        vb = np.ascontiguousarray(vp[pages][:, :, kvh:kvh + 1])
        t0, t1 = int(cu[b]), int(cu[b + 1])
        tic = time.perf_counter()
        oracle.attention_ref(q[t0:t1, h:h + 1], kb, vb, np.arange(n, dtype=np.int32)[None],
                             [L], [0, t1 - t0], c.scale, True, c.page_size)
        t_used += time.perf_counter() - tic
        flops += units.prefill_flops([L], [t1 - t0], 1, c.D, True)
        done += 1
        if t_used >= min_s:
            break
    return {"value": flops / t_used / 1e9, "unit": "GFLOP/s", "cores": cores,
            "blas_threads": blas, "kind": "oracle",
            "sample": f"{c.name}: {done} of the {len(planes)} (sequence, query head) planes "
                      f"({t1 - t0} causal rows over {L} keys each), float64 NumPy with the "
                      f"scores materialised, {t_used:.1f} s of oracle time"}


# ---------------------------------------------------------------------------

class PreparedStep:
    """A step's C calls replayed through pa.prepared(): the arguments are marshalled
    once and no Python-side checks run per call, as in a launch loop whose host cost
    matters (the tiny decode is bound by it)."""

    def __init__(self, step):
        self.step = step
        self.units, self.unit_name = step.units, step.unit_name
        self.run = step.pa.prepared(step)

    def __call__(self):
        self.run()

    def config(self):
        cfg = dict(self.step.config())
        cfg["launch"] = "pa.prepared: C calls replayed with marshalled arguments"
        return cfg


def secondary_figure(label, name, splits, args):
    """One secondary line: the workload `name` timed like the headline (a HIP graph
    replay when the label ends in _graph)."""
    s = make_step(name, splits)
    if label.endswith("_graph"):
        s = GraphStep(s, len(s.kv) if hasattr(s, "kv") else 1)
    elif label.endswith("_prepared"):
        s = PreparedStep(s)
    w2, e2, k2 = time_step(s, args.steps, args.warmup, settle_ms=SECONDARY_SETTLE_MS)
    v2 = rate(s.units, e2, s.unit_name)
    pk = HBM_PEAK_GBS if s.unit_name == "GB/s" else BF16_PEAK_TFLOPS
    per = getattr(s, "calls", 1)
    fig = {"value": round(v2, 2), "unit": s.unit_name, "frac": round(v2 / pk, 4),
           "us_per_step": round(e2 * 1e3 / per, 2), "settle_ms": SECONDARY_SETTLE_MS,
           "config": s.config()}
    if k2:
        fig["main_kernel_us"] = round(k2 * 1e3, 2)
        fig["main_kernel_frac"] = round(rate(s.units, k2, s.unit_name) / pk, 4)
    log(f"[bench] {label}: {e2 * 1e3 / per:.1f} us/step, {v2:.2f} {s.unit_name}")
    return fig


def dominant_kernel_name(workload, bound):
    """The dominant kernel's name: the profiler name recorded for the workload, else the
    decode partition kernel (HBM-bound steps) or the prefill kernel."""
    if workload in TRAFFIC:
        return TRAFFIC[workload][2].split("::")[-1].rstrip("<")
    return "decode_partition_kernel" if bound == "hbm" else "prefill_kernel"


def roofline_object(step, workload, kern_ms, ev_ms):
    """The roofline of a step's dominant kernel: algorithmic units per launch over the
    kernel's own (dispatch-stamped) duration against MI355X's published peak, with
    the counter-measured HBM traffic recorded for the same sources (or null)."""
    bound = "hbm" if step.unit_name == "GB/s" else "mfma"
    peak = HBM_PEAK_GBS if bound == "hbm" else BF16_PEAK_TFLOPS
    if kern_ms is None:                      # the mixed step: no single main kernel
        kern_ms = ev_ms
    achieved = rate(step.units, kern_ms, step.unit_name)
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak,
            "unit": step.unit_name, "frac": round(achieved / peak, 4),
            "traffic": recorded_traffic(workload),
            "algorithmic_units_per_launch": int(step.units),
            "kernel": dominant_kernel_name(workload, bound)
            if not isinstance(step, MixedStep) else "whole step",
            "kernel_us_per_launch": round(kern_ms * 1e3, 2),
            "kernel_us_median": round(getattr(step, "kernel_ms_median", kern_ms) * 1e3, 2),
            "kernel_us_min": round(getattr(step, "kernel_ms_min", kern_ms) * 1e3, 2),
            "kernel_timing": "start/end events stamped by that kernel's own dispatch "
                             "(hipExtLaunchKernel) in a second pass of the same steps "
                             "right after the timed pass",
            "step_us": round(ev_ms * 1e3, 2)}


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(args.workload, args.record_traffic)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the multi-GPU "
                                   "sharding of the path is described, not built",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import paged_kv_flashattention_amd as pa
    pa.load_library()
    torch.cuda.init()
    log(f"[bench] device {torch.cuda.get_device_name(0)}; workload {args.workload}")

    if args.traffic_pass:
        traffic_pass(args.steps, args.workload)
        return

    step = make_step(args.workload, args.num_splits)
    torch.cuda.synchronize()
    wall, ev, kern_ms = time_step(step, args.steps, args.warmup, settle_ms=args.settle_ms)
    value = rate(step.units, ev, step.unit_name)
    launch = pa.describe_launch()
    if kern_ms is None:                      # the mixed step: no single main kernel
        kern_ms = ev
    achieved = rate(step.units, kern_ms, step.unit_name)
    log(f"[bench] {args.workload}: {ev * 1e3:.1f} us/step (events), {wall * 1e3:.1f} us/step "
        f"(wall), {value:.1f} {step.unit_name}; dominant kernel {kern_ms * 1e3:.1f} us, "
        f"{achieved:.1f} {step.unit_name}; {launch}")
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": step.unit_name,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall, 5),
        **({"settle_ms": args.settle_ms} if args.settle_ms > 0 else {}),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": step.config(),
        "roofline": roofline_object(step, args.workload, kern_ms, ev),
    }
    bound = result["roofline"]["bound"]
    del step
    torch.cuda.empty_cache()
    if bound == "hbm":
        read_gbs, read_blocks = stream_read_gbs()
        result["roofline"]["measured_read_GBs"] = round(read_gbs, 1)
        result["roofline"]["frac_of_measured_read"] = round(achieved / read_gbs, 4)
        log(f"[bench] streaming read of {STREAM_BYTES >> 30} GiB: {read_gbs:.1f} GB/s "
            f"({read_blocks} work-groups); the dominant kernel reaches "
            f"{achieved / read_gbs:.1%} of it")

    if not args.no_secondary and args.workload == "qwen7b_decode":
        # the metric's second half: causal prefill (4 x 4096, Hq 32, Hkv 8) with a
        # roofline object of its own and its own oracle baseline
        try:
            pf = make_step("causal_prefill", 0)
            w2, e2, k2 = time_step(pf, args.steps, args.warmup,
                                   settle_ms=SECONDARY_SETTLE_MS)
            result["roofline_prefill"] = dict(roofline_object(pf, "causal_prefill", k2, e2),
                                              value=round(rate(pf.units, e2, pf.unit_name), 2),
                                              settle_ms=SECONDARY_SETTLE_MS,
                                              config=pf.config())
            log(f"[bench] causal_prefill: {e2 * 1e3:.1f} us/step, kernel {k2 * 1e3:.1f} us, "
                f"{result['roofline_prefill']['achieved']:.1f} TFLOP/s in the kernel")
            if not args.no_cpu_baseline:
                cb = cpu_baseline(pf)
                result["cpu_baseline_prefill"] = cb
                log(f"[bench] prefill cpu baseline: {cb['value']:.3f} {cb['unit']} "
                    f"({cb['sample']})")
            del pf
        except Exception as exc:                          # noqa: BLE001
            result["roofline_prefill"] = {"error": f"{type(exc).__name__}: {exc}"}
            log(f"[bench] causal_prefill: failed ({type(exc).__name__}: {exc})")
        torch.cuda.empty_cache()
        # the other workloads, same timing; the long-context decode both with the 64
        # partitions it is stated with and with the library's own split choice; the C2
        # decode and the mixed step also replayed from a HIP graph (*_graph)
        extra = {}
        for label, name, splits in (("qwen7b_decode_graph", "qwen7b_decode", 0),
                                    ("qwen7b_decode_warm", "qwen7b_decode_warm", 0),
                                    ("tiny_decode", "tiny_decode", 0),
                                    ("tiny_decode_prepared", "tiny_decode", 0),
                                    ("qwen7b_decode_fp8", "qwen7b_decode_fp8", 0),
                                    ("causal_prefill_fp8", "causal_prefill_fp8", 0),
                                    ("causal_prefill_block_map", "causal_prefill_block_map", 0),
                                    ("long_decode", "long_decode", 64),
                                    ("long_decode_auto_splits", "long_decode", -1),
                                    ("long_history_chunk", "long_history_chunk", 0),
                                    ("mixed_ragged", "mixed_ragged", 0),
                                    ("mixed_ragged_graph", "mixed_ragged", 0),
                                    ("mixed_ragged_two_streams", "mixed_ragged_two_streams", 0)):
            # a secondary workload that fails is reported as such; the headline stands
            try:
                if splits < 0:
                    from workloads import make_config
                    c = make_config(name, "cuda")
                    splits = pa.decode_num_splits(c.B, c.Hkv, c.max_seq_len)
                    del c
                extra[label] = secondary_figure(label, name, splits, args)
            except Exception as exc:                      # noqa: BLE001
                extra[label] = {"error": f"{type(exc).__name__}: {exc}"}
                log(f"[bench] {label}: failed ({type(exc).__name__}: {exc})")
            torch.cuda.empty_cache()
        result["secondary"] = extra

    if not args.no_cpu_baseline:
        try:
            s = make_step(args.workload, args.num_splits)
            cb = cpu_baseline(s)
            del s
        except Exception as exc:                          # noqa: BLE001
            cb = None
            result["cpu_baseline"] = {"error": f"{type(exc).__name__}: {exc}"}
            log(f"[bench] cpu baseline failed ({type(exc).__name__}: {exc})")
        if cb is not None:
            result["cpu_baseline"] = cb
            log(f"[bench] cpu baseline: {cb['value']:.3f} {cb['unit']} ({cb['sample']})")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
