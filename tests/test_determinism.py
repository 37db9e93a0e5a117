"""Run-to-run determinism, and one run with every launch made blocking.

No kernel here uses atomics or an order of accumulation that depends on timing, so the
same inputs must give the same bits on every run; a difference would mean a missing
wait or barrier, i.e. a race whose outcome depends on scheduling ("The Stack Below the
Stack (Part 2)", section 2: a missing barrier makes results depend on the schedule).
The same outputs are then produced once more in a fresh process with
HIP_LAUNCH_BLOCKING=1 (every launch completes before the next is issued) and compared
bit for bit.
"""

import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest
import torch

import paged_kv_flashattention_amd as pa
from workloads import bits, make_case, random_e4m3_codes

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def outputs():
    """Prefill of three causal chunks over history (8-wave work-groups, in one pass and
    with 4 key parts), the same over FP8 pools, and a 6-split decode of four sequences,
    all from fixed seeds; returns host arrays (bf16 as uint16 bits, lse as float32)."""
    pf = make_case("detp", hist_lens=[3000, 0, 200], q_lens=[600, 1100, 64], write_new=True,
                   causal=True, Hq=8, Hkv=2, D=128, page_size=16, seed=41, device="cuda")
    pa.kv_page_write(pf.k_pool, pf.v_pool, pf.k_new, pf.v_new, pf.cu_new, pf.start_pos,
                     pf.block_tables)
    args = (pf.q, pf.k_pool, pf.v_pool, pf.cu_seqlens_q, pf.seq_lens_k, pf.block_tables,
            pf.scale)
    o1, l1 = pa.paged_attn_prefill_varlen(*args, causal=True, max_q_len=1100, return_lse=True)
    o4, l4 = pa.paged_attn_prefill_varlen_splitk(*args, causal=True, max_q_len=1100,
                                                 num_splits=4, return_lse=True)
    shape = tuple(pf.k_pool.shape)
    kc, vc = random_e4m3_codes(shape, 42, "cuda"), random_e4m3_codes(shape, 43, "cuda")
    o8, l8 = pa.paged_attn_prefill_varlen_fp8(pf.q, kc, vc, pf.cu_seqlens_q, pf.seq_lens_k,
                                              pf.block_tables, pf.scale, 0.03, 0.05,
                                              causal=True, max_q_len=1100, return_lse=True)
    dc = make_case("detd", seq_lens=[3000, 17, 999, 4096], Hq=28, Hkv=4, D=128, page_size=16,
                   seed=4, device="cuda")
    od, ld = pa.paged_attn_decode(dc.q, dc.k_pool, dc.v_pool, dc.block_tables, dc.seq_lens_k,
                                  dc.scale, max_seq_len=4096, num_splits=6, return_lse=True)
    torch.cuda.synchronize()
    host = lambda t: t.cpu().numpy()                                           # noqa: E731
    return {"o1": bits(o1), "l1": host(l1), "o4": bits(o4), "l4": host(l4),
            "o8": bits(o8), "l8": host(l8), "od": bits(od), "ld": host(ld)}


def _same(a, b):
    assert a.keys() == b.keys()
    for k in a:
        # bitwise, NaN-free by construction (every row here sees at least one key)
        assert np.array_equal(a[k].view(np.uint32 if a[k].dtype == np.float32 else np.uint16),
                              b[k].view(np.uint32 if b[k].dtype == np.float32 else np.uint16)), k


def test_repeat_runs_are_bitwise_identical(require_gpu):
    print("[determinism] prefill (one pass, 4 parts, FP8) and decode, 10 runs", flush=True)
    ref = outputs()
    for _ in range(9):
        _same(outputs(), ref)


def test_blocking_launches_give_the_same_bits(require_gpu):
    ref = outputs()
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "blocking.npz")
        code = ("import sys; sys.path.insert(0, %r); import numpy as np; "
                "from tests.test_determinism import outputs; np.savez(%r, **outputs())"
                % (ROOT, path))
        env = dict(os.environ, HIP_LAUNCH_BLOCKING="1")
        print("[determinism] the same outputs in a process with HIP_LAUNCH_BLOCKING=1",
              flush=True)
        res = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT,
                             capture_output=True, text=True, timeout=300)
        assert res.returncode == 0, res.stderr[-3000:]
        with np.load(path) as z:
            got = {k: z[k] for k in z.files}
    _same(got, ref)
