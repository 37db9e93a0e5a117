"""The C-ABI boundary: the library loads, exports what the header declares, and
rejects invalid arguments with the documented status before touching a GPU."""

import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attn.h")


@pytest.fixture(scope="module")
def lib():
    from paged_kv_flashattention_amd import _lib, build
    if not os.path.exists(_lib.LIB_PATH):
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) -
                  {"if", "sizeof", "defined"})


def test_header_declares_the_four_operations():
    names = declared_functions()
    for n in ["kv_page_write", "paged_attn_decode", "paged_attn_splitk_reduce",
              "paged_attn_prefill_varlen", "kv_page_write_fp8", "paged_attn_decode_fp8",
              "paged_attn_prefill_varlen_splitk", "paged_attn_prefill_num_splits",
              "paged_attn_prefill_plan_splits",
              "paged_attn_prefill_workspace_bytes", "paged_attn_decode_ex",
              "paged_attn_decode_ex_workspace_bytes", "paged_attn_prefill_ex",
              "paged_attn_prefill_ex_workspace_bytes", "paged_attn_decode_workspace_bytes",
              "paged_attn_decode_num_splits", "pa_status_string", "pa_last_error",
              "pa_describe_launch"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    from paged_kv_flashattention_amd import _lib
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding lacks a signature for {name}"


def test_status_strings(lib):
    assert lib.pa_status_string(0) == b"PA_OK"
    assert lib.pa_status_string(3) == b"PA_ERR_UNSUPPORTED"
    assert lib.pa_status_string(99) == b"PA_ERR_UNKNOWN"


FAKE = 0x10000          # 16-byte aligned non-null address; never dereferenced on these paths


def decode_call(lib, **over):
    args = dict(out=FAKE, lse=None, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, B=2,
                max_pages=4, num_pages=8, ps=16, Hq=8, Hkv=2, D=128, scale=0.1, max_seq=64,
                S=1, ws=None, ws_bytes=0)
    args.update(over)
    return lib.paged_attn_decode(args["out"], args["lse"], args["q"], args["k"], args["v"],
                                 args["bt"], args["lens"], args["B"], args["max_pages"],
                                 args["num_pages"], args["ps"], args["Hq"], args["Hkv"],
                                 args["D"], args["scale"], args["max_seq"], args["S"],
                                 args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(q=None), 1),
    (dict(bt=None), 1),
    (dict(D=96), 3),
    (dict(ps=24), 3),
    (dict(Hq=7, Hkv=2), 3),
    (dict(Hq=34, Hkv=2), 3),            # group of 17
    (dict(B=-1), 2),
    (dict(num_pages=0), 2),
    (dict(q=FAKE + 8), 4),
    (dict(S=4, ws=None), 5),
    (dict(S=4, ws=FAKE, ws_bytes=16), 5),
    (dict(scale=float("nan")), 2),
    (dict(scale=0.0), 2),
    (dict(scale=-0.1), 2),
    (dict(scale=float("inf")), 2),
])
def test_decode_rejects_invalid_arguments(lib, over, status):
    assert decode_call(lib, **over) == status
    assert lib.pa_last_error() != b""


def test_decode_with_no_sequences_is_ok(lib):
    assert decode_call(lib, B=0, out=None, q=None) in (0, 1)


def test_workspace_sizing(lib):
    assert lib.paged_attn_decode_workspace_bytes(32, 28, 4, 128, 8192, 1) == 0
    need = lib.paged_attn_decode_workspace_bytes(32, 28, 4, 128, 8192, 8)
    rows = 32 * 28 * 8
    assert need >= rows * 128 * 4 + rows * 4
    auto = lib.paged_attn_decode_num_splits(32, 4, 8192)
    assert 1 <= auto <= 8192 // 32
    assert lib.paged_attn_decode_num_splits(1, 1, 10) == 1        # one chunk -> one split
    # split count never exceeds the number of 32-key chunks
    assert lib.paged_attn_decode_workspace_bytes(1, 4, 4, 128, 100, 64) == \
        lib.paged_attn_decode_workspace_bytes(1, 4, 4, 128, 100, 4)


def test_prefill_and_write_reject_invalid_arguments(lib):
    f = lib.paged_attn_prefill_varlen
    base = [FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 10, 8, 4, 8, 16, 8, 2, 128,
            0.1, 1, None]
    assert f(*base) == 0 or True   # valid arguments are not launched here (no GPU)
    bad = list(base); bad[2] = None
    assert f(*bad) == 1
    bad = list(base); bad[16] = 80
    assert f(*bad) == 3
    bad = list(base); bad[13] = 48
    assert f(*bad) == 3
    bad = list(base); bad[0] = FAKE + 2
    assert f(*bad) == 4
    w = lib.kv_page_write
    wb = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 10, 4, 8, 16, 2, 128, None]
    bad = list(wb); bad[4] = None
    assert w(*bad) == 1
    bad = list(wb); bad[11] = 8
    assert w(*bad) == 3
    bad = list(wb); bad[8] = 0
    assert w(*bad) == 0          # nothing to write
    r = lib.paged_attn_splitk_reduce
    assert r(FAKE, None, FAKE, FAKE, 4, 0, 128, None) == 2
    assert r(FAKE, None, FAKE, FAKE, 4, 2, 32, None) == 3
    assert r(None, None, FAKE, FAKE, 4, 2, 128, None) == 1


def decode_fp8_call(lib, ks=0.01, vs=0.02, **over):
    args = dict(out=FAKE, lse=None, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, B=2,
                max_pages=4, num_pages=8, ps=16, Hq=8, Hkv=2, D=128, scale=0.1, max_seq=64,
                S=1, ws=None, ws_bytes=0)
    args.update(over)
    return lib.paged_attn_decode_fp8(args["out"], args["lse"], args["q"], args["k"], args["v"],
                                     args["bt"], args["lens"], args["B"], args["max_pages"],
                                     args["num_pages"], args["ps"], args["Hq"], args["Hkv"],
                                     args["D"], args["scale"], ks, vs, args["max_seq"],
                                     args["S"], args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("ks,vs,over,status", [
    (0.0, 0.02, {}, 2),
    (0.01, -1.0, {}, 2),
    (float("nan"), 0.02, {}, 2),
    (0.01, float("inf"), {}, 2),
    (3.0e38, 0.02, dict(scale=10.0), 2),        # softmax_scale * k_scale overflows
    (0.01, 0.02, dict(k=None), 1),
    (0.01, 0.02, dict(D=96), 3),
    (0.01, 0.02, dict(v=FAKE + 4), 4),
    (0.01, 0.02, dict(S=4, ws=FAKE, ws_bytes=16), 5),
])
def test_decode_fp8_rejects_invalid_arguments(lib, ks, vs, over, status):
    assert decode_fp8_call(lib, ks, vs, **over) == status
    assert lib.pa_last_error() != b""


def test_write_fp8_rejects_invalid_arguments(lib):
    w = lib.kv_page_write_fp8
    wb = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 10, 4, 8, 16, 2, 128, 0.5, 0.25, None]
    for i, v, st in [(14, 0.0, 2), (15, float("nan"), 2), (15, -2.0, 2), (14, float("inf"), 2),
                     (4, None, 1), (11, 8, 3), (1, FAKE + 8, 4)]:
        bad = list(wb); bad[i] = v
        assert w(*bad) == st, (i, v)
    bad = list(wb); bad[8] = 0
    assert w(*bad) == 0          # nothing to write
    assert b"nothing" in lib.pa_describe_launch()


def test_prefill_splitk_sizing_and_rejections(lib):
    n = lib.paged_attn_prefill_num_splits
    assert n(4, 32, 4096) == 1          # 2048 work-groups of 256 rows fill the chip
    assert n(5, 32, 512) == 1           # 640 work-groups of 128 rows fill 512 slots
    assert n(1, 32, 512) == 4           # 128 work-groups: one per slot with 4 parts
    assert n(1, 1, 100) == 8            # at most 8 automatically
    wb = lib.paged_attn_prefill_workspace_bytes
    assert wb(1, 512, 512, 32, 128, 1) == 0
    need = wb(1, 512, 512, 32, 128, 4)
    assert need >= 512 * 32 * 4 * 129 * 4
    assert wb(1, 512, 512, 32, 128, 0) == need          # auto resolves to the same 4
    assert wb(1, 512, 512, 32, 128, 99) == wb(1, 512, 512, 32, 128, 16)   # capped at 16
    f = lib.paged_attn_prefill_varlen_splitk
    base = [FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 512, 512, 2100, 2100, 16, 32, 8,
            128, 0.1, 1, 4, None, 0, None]
    assert f(*base) == 5                                  # workspace missing
    bad = list(base); bad[20] = FAKE; bad[21] = 16
    assert f(*bad) == 5                                   # workspace too small
    bad = list(base); bad[20] = FAKE + 4; bad[21] = need
    assert f(*bad) == 4                                   # workspace misaligned
    bad = list(base); bad[16] = 96
    assert f(*bad) == 3
    bad = list(base); bad[9] = 0
    assert f(*bad) == 0 and b"nothing" in lib.pa_describe_launch()


def test_options_entry_points_check_their_options(lib):
    from paged_kv_flashattention_amd import _lib
    d = lib.paged_attn_decode_ex
    args = [FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 8, 16, 8, 2, 128, 0.1, 64]
    assert d(*args, None, None, 0, None) == 1                         # NULL opts
    bad = _lib.DecodeOpts(1, -3, 0, 1.0, 1.0)
    assert d(*args, ctypes.byref(bad), None, 0, None) == 2            # negative window
    bad = _lib.DecodeOpts(1, 0, 2, 1.0, 1.0)
    assert d(*args, ctypes.byref(bad), None, 0, None) == 3            # unknown pool format
    bad = _lib.DecodeOpts(1, 0, 1, 0.0, 1.0)
    assert d(*args, ctypes.byref(bad), None, 0, None) == 2            # FP8 scale 0
    wb = lib.paged_attn_decode_ex_workspace_bytes
    plain = _lib.DecodeOpts(8, 0, 0, 1.0, 1.0)
    win = _lib.DecodeOpts(8, 100, 0, 1.0, 1.0)
    assert wb(32, 28, 4, 128, 8192, ctypes.byref(plain)) == \
        lib.paged_attn_decode_workspace_bytes(32, 28, 4, 128, 8192, 8)
    # a 100-key window walks at most 131 keys: 5 chunks, so at most 5 splits
    assert wb(32, 28, 4, 128, 8192, ctypes.byref(win)) == \
        lib.paged_attn_decode_workspace_bytes(32, 28, 4, 128, 8192, 5)
    assert wb(32, 28, 4, 128, 8192, None) == 0
    p = lib.paged_attn_prefill_ex
    pargs = [FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 10, 8, 4, 8, 16, 8, 2, 128, 0.1]
    assert p(*pargs, None, None, 0, None) == 1
    bad = _lib.PrefillOpts(1, -1, 1)
    assert p(*pargs, ctypes.byref(bad), None, 0, None) == 2
    assert lib.paged_attn_prefill_ex_workspace_bytes(1, 512, 512, 32, 128, None) == 0
    po = _lib.PrefillOpts(1, 64, 4)
    assert lib.paged_attn_prefill_ex_workspace_bytes(1, 512, 512, 32, 128, ctypes.byref(po)) == \
        lib.paged_attn_prefill_workspace_bytes(1, 512, 512, 32, 128, 4)


def test_page_scale_options_are_checked(lib):
    """FP8 scales per (page, KV head): both arrays or neither, FP8 pools only, 4-byte
    aligned; the page write's own entry point needs both; prefill does not combine
    them with ALiBi slopes."""
    from paged_kv_flashattention_amd import _lib
    d = lib.paged_attn_decode_ex
    args = [FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 8, 16, 8, 2, 128, 0.1, 64]
    ws = lib.paged_attn_decode_ex_workspace_bytes(2, 8, 2, 128, 64, None)
    for fmt, ks, vs, st in [(1, FAKE, None, 1), (1, None, FAKE, 1), (0, FAKE, FAKE, 3),
                            (1, FAKE + 2, FAKE, 4), (1, FAKE, FAKE + 1, 4)]:
        o = _lib.DecodeOpts(1, 0, fmt, 1.0, 1.0)
        o.k_scales, o.v_scales = ks, vs
        assert d(*args, ctypes.byref(o), None, ws, None) == st, (fmt, ks, vs)
        assert b"scales" in lib.pa_last_error()
    p = lib.paged_attn_prefill_ex
    pargs = [FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 10, 8, 4, 8, 16, 8, 2, 128, 0.1]
    o = _lib.PrefillOpts(1, 0, 1)
    o.kv_fp8, o.k_scale, o.v_scale, o.k_scales, o.v_scales = 1, 1.0, 1.0, FAKE, FAKE
    o.alibi_slopes = FAKE
    assert p(*pargs, ctypes.byref(o), None, 0, None) == 3
    o.k_scales = None
    assert p(*pargs, ctypes.byref(o), None, 0, None) == 1
    w = lib.kv_page_write_fp8_scales
    wb = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 10, 4, 8, 16, 2, 128, FAKE, FAKE, None]
    for i, v, st in [(14, None, 1), (15, None, 1), (14, FAKE + 2, 4), (11, 8, 3), (4, None, 1)]:
        bad = list(wb); bad[i] = v
        assert w(*bad) == st, (i, v)
    bad = list(wb); bad[8] = 0
    assert w(*bad) == 0 and b"nothing" in lib.pa_describe_launch()


def test_binding_takes_page_scales_as_tensor_pairs():
    import paged_kv_flashattention_amd as pa
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    k8 = torch.zeros(4, 16, 2, 128, dtype=torch.uint8)
    bt = torch.zeros(2, 2, dtype=torch.int32)
    lens = torch.zeros(2, dtype=torch.int32)
    sc = torch.ones(4, 2, dtype=torch.float32)
    with pytest.raises(TypeError):       # a float and a tensor do not mix
        pa.paged_attn_decode_fp8(q, k8, k8, bt, lens, 0.1, sc, 0.5)
    with pytest.raises(TypeError):       # scales are float32
        pa.paged_attn_decode_fp8(q, k8, k8, bt, lens, 0.1, sc.double(), sc.double())


def test_block_map_options_are_checked(lib):
    """Block maps: positive dimensions, no key parts, at most 262144 keys per sequence;
    no workspace."""
    from paged_kv_flashattention_amd import _lib
    p = lib.paged_attn_prefill_ex
    pargs = [FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 10, 8, 4, 8, 16, 8, 2, 128, 0.1]

    def opts(**kw):
        o = _lib.PrefillOpts(1, 0, 1)
        o.block_map, o.block_map_q_blocks, o.block_map_k_blocks = FAKE, 1, 2
        for k, v in kw.items():
            setattr(o, k, v)
        return o
    for kw, st in [(dict(block_map_q_blocks=0), 2), (dict(block_map_k_blocks=-1), 2),
                   (dict(num_splits=2), 3), (dict(kv_fp8=1, k_scale=1.0, v_scale=1.0,
                                                  num_splits=2), 3)]:
        o = opts(**kw)
        assert p(*pargs, ctypes.byref(o), None, 0, None) == st, kw
        assert b"block map" in lib.pa_last_error()
    big = list(pargs)
    big[11] = 20000                                           # 20000 pages of 16 keys
    o = opts()
    assert p(*big, ctypes.byref(o), None, 0, None) == 3
    o = opts(num_splits=0)
    assert lib.paged_attn_prefill_ex_workspace_bytes(1, 512, 512, 32, 128, ctypes.byref(o)) == 0


def test_binding_refuses_a_negative_window():
    import paged_kv_flashattention_amd as pa
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    kp = torch.zeros(4, 16, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pa.paged_attn_decode(q, kp, kp, torch.zeros(2, 2, dtype=torch.int32),
                             torch.zeros(2, dtype=torch.int32), 0.1, window_left=-1)


def test_binding_refuses_wrong_dtypes_before_any_device_work():
    import paged_kv_flashattention_amd as pa
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    kp = torch.zeros(4, 16, 2, 128, dtype=torch.bfloat16)
    bt64 = torch.zeros(2, 2, dtype=torch.int64)
    lens = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(TypeError):
        pa.paged_attn_decode(q, kp, kp, bt64, lens, 0.1)
    with pytest.raises(TypeError):
        pa.paged_attn_decode(q.half(), kp, kp, bt64.int(), lens, 0.1)
    with pytest.raises(TypeError):
        pa.paged_attn_prefill_varlen(q, kp.float(), kp, lens, lens, bt64.int(), 0.1)
    with pytest.raises(ValueError):      # a CPU tensor is refused, never computed on
        pa.paged_attn_decode(q, kp, kp, bt64.int(), lens, 0.1)
    with pytest.raises(TypeError):       # FP8 entry points take code pools only
        pa.paged_attn_decode_fp8(q, kp, kp, bt64.int(), lens, 0.1, 0.01, 0.01)
    k8 = torch.zeros(4, 16, 2, 128, dtype=torch.uint8)
    with pytest.raises(ValueError):      # scales are checked before anything else runs
        pa.paged_attn_decode_fp8(q, k8, k8, bt64.int(), lens, 0.1, 0.0, 0.01)
    with pytest.raises(ValueError):
        pa.paged_attn_decode_fp8(q, k8, k8, bt64.int(), lens, 0.1, 0.01, 0.01)   # CPU pools
    kn = torch.zeros(3, 2, 128, dtype=torch.bfloat16)
    cu = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(TypeError):
        pa.kv_page_write_fp8(kp, kp, kn, kn, cu, lens, bt64.int(), 0.1, 0.1)
    with pytest.raises(TypeError):
        pa.kv_page_write_fp8(k8, k8, kn.float(), kn, cu, lens, bt64.int(), 0.1, 0.1)


@pytest.mark.gpu
def test_describe_launch_names_the_kernel(require_gpu):
    import paged_kv_flashattention_amd as pa
    from workloads import make_case
    case = make_case("d", seq_lens=[100, 50], Hq=8, Hkv=2, D=128, page_size=16, seed=1,
                     device="cuda")
    pa.paged_attn_decode(case.q, case.k_pool, case.v_pool, case.block_tables, case.seq_lens_k,
                         case.scale, max_seq_len=100, num_splits=2)
    torch.cuda.synchronize()
    d = pa.describe_launch()
    assert "decode_partition" in d and "splits=2" in d


@pytest.mark.gpu
def test_failed_call_leaves_output_untouched(require_gpu):
    import paged_kv_flashattention_amd as pa
    from workloads import make_case
    case = make_case("d", seq_lens=[100, 50], Hq=8, Hkv=2, D=128, page_size=16, seed=1,
                     device="cuda")
    out = torch.full((2, 8, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(pa.PagedAttnError) as e:
        pa.paged_attn_decode(case.q, case.k_pool, case.v_pool, case.block_tables,
                             case.seq_lens_k, case.scale, max_seq_len=100, num_splits=3,
                             out=out, workspace=ws)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert (out.float() == 7.0).all()


def _tiles_model(q_lens, k_lens, causal, window):
    """Per-query-tile 64-key counts, restated from the kernel's documented bounds:
    a tile of R rows (R = 256 when the longest query run reaches 512, else 128)
    whose last row sits at position p_last needs keys 0 .. p_last (all keys without
    causal), and with a window w its first row's window starts at p_first - w + 1."""
    R = 256 if max(q_lens) >= 512 else 128
    out = []
    for q, L in zip(q_lens, k_lens):
        for r0 in range(0, q, R):
            r1 = min(q, r0 + R)                       # one past the tile's last row
            last_key = L - q + r1 if causal else L    # keys [0, last_key)
            last_key = max(0, min(L, last_key))
            n = -(-last_key // 64)
            first = 0
            if window > 0:
                first = min(max(0, L - q + r0 - window + 1) // 64, n)
            out.append(n - first)
    return out, 256 * (8 * 32 // R)


def _makespan(tiles, Hq, s, slots):
    """Heaviest-first list scheduling of the work-groups of part count s onto the
    slots: each (tile, head) cut into p = min(s, tiles // 16) (at least 1) parts of
    consecutive key tiles, each work-group charged 2 extra tiles, the merge 3."""
    import heapq
    jobs, cut = [], False
    for t in tiles:
        p = max(1, min(s, t // 16)) if s > 1 else 1
        cut |= p > 1
        jobs += [(k + 1) * t // p - k * t // p + 2 for k in range(p)] * Hq
    loads = [0] * slots
    for j in sorted(jobs, reverse=True):
        heapq.heappush(loads, heapq.heappop(loads) + j)
    return max(loads) + (3 if cut else 0)


def _plan_model(q_lens, k_lens, Hq, causal, window):
    if not q_lens or max(q_lens) == 0:
        return 1
    tiles, slots = _tiles_model(q_lens, k_lens, causal, window)
    heavy, work = max(tiles), sum(tiles) * Hq
    if heavy < 32 or heavy * slots <= work:
        return 1
    # ceil(heavy / mean - 0.05), mean = work / slots
    s_lo = max(1, -(-(20 * heavy * slots - work) // (20 * work)))
    if s_lo > 8:
        return 8
    if len(tiles) * Hq > 1 << 14:
        return s_lo
    cost = {s: _makespan(tiles, Hq, s, slots) for s in range(s_lo, 9)}
    best = min(cost.values())
    return min(s for s, c in cost.items() if c * 100 <= best * 103)


def test_prefill_plan_splits_null_arrays(lib):
    assert lib.paged_attn_prefill_plan_splits(2, None, None, 8, 1, 0) == 0
    assert b"NULL" in lib.pa_last_error()
    assert lib.paged_attn_prefill_plan_splits(0, None, None, 8, 1, 0) == 1


def test_prefill_plan_splits_host_logic():
    """The planner (host code, no GPU) against a restatement of its rule on fixed
    and random batches, its documented special cases, and its rejections."""
    import numpy as np
    import paged_kv_flashattention_amd as pa
    from paged_kv_flashattention_amd import PagedAttnError
    # a full grid of equal causal rows needs no parts
    assert pa.prefill_plan_splits([4096] * 4, [4096] * 4, 32) == 1
    # 5 chunks of 512 over histories 214 .. 4,113 (256-row tiles, two per chunk): the
    # heaviest tile (73 key tiles) is 2.0 times the mean load per slot; 2 parts bring
    # the modelled makespan from 75 to 44 tiles, more parts do not lower it (3: 53)
    assert pa.prefill_plan_splits([512] * 5, [1732, 726, 4625, 1703, 850], 32) == 2
    # one chunk over a long history: 64 work-groups of ~520 tiles on 256 slots --
    # 4 parts fill the slots once; 5 would need a second round for 64 of them
    assert pa.prefill_plan_splits([512], [33280], 32) == 4
    assert pa.prefill_plan_splits([512], [33280], 1) == 8           # capped at 8
    assert pa.prefill_plan_splits([512], [600], 1) == 1             # too short to cut
    assert pa.prefill_plan_splits([], [], 32) == 1
    assert pa.prefill_plan_splits([0, 0], [100, 5], 32) == 1
    rng = np.random.default_rng(7)
    for _ in range(60):
        B = int(rng.integers(1, 7))
        q = [int(x) for x in rng.integers(0, 1500, B)]
        h = [int(x) for x in rng.integers(0, 40000, B)]
        k = [a + b for a, b in zip(q, h)]
        Hq = int(rng.choice([1, 4, 8, 32]))
        causal = bool(rng.integers(0, 2))
        window = int(rng.choice([0, 0, 100, 3000]))
        got = pa.prefill_plan_splits(q, k, Hq, causal=causal, window_left=window)
        assert got == _plan_model(q, k, Hq, causal, window), (q, k, Hq, causal, window)
        assert 1 <= got <= 8
    for q, k in (([1], [-1]), ([-3], [10])):
        with pytest.raises(PagedAttnError):
            pa.prefill_plan_splits(q, k, 32)
    with pytest.raises(PagedAttnError):
        pa.prefill_plan_splits([1], [1], 0)
    with pytest.raises(ValueError):
        pa.prefill_plan_splits([1], [1], 8, window_left=-1)


def test_mixed_step_arguments_are_checked(lib):
    """paged_attn_mixed: NULL parts, each part checked as its own entry point checks it
    (the message names the part), empty parts skipped, and the workspace sized as the
    prefill's key parts (256-row tiles) plus the decode's partials; nothing here
    reaches a launch."""
    from paged_kv_flashattention_amd import _lib
    m = lib.paged_attn_mixed
    w = lib.paged_attn_mixed_workspace_bytes
    P, ps, Hq, Hkv, D = 64, 16, 8, 2, 128

    def pf(**kw):
        p = _lib.MixedPrefill(FAKE, None, FAKE, FAKE, FAKE, FAKE, 2, 1200, 600, 8, 1, 3)
        for k, v in kw.items():
            setattr(p, k, v)
        return p

    def dec(**kw):
        d = _lib.MixedDecode(FAKE, None, FAKE, FAKE, FAKE, 3, 8, 120, 2)
        for k, v in kw.items():
            setattr(d, k, v)
        return d
    args = (FAKE, FAKE, P, ps, Hq, Hkv, D, 0.1)
    assert m(None, ctypes.byref(dec()), None, *args, None, 0, None) == 1
    assert m(ctypes.byref(pf()), None, None, *args, None, 0, None) == 1
    # both parts empty: nothing to do, nothing checked
    assert m(ctypes.byref(pf(B=0, cu_seqlens_q=None)), ctypes.byref(dec(B=0, q=None)), None,
             *args, None, 0, None) == 0
    assert b"nothing to do" in lib.pa_describe_launch()
    # a missing pointer or a bad size in one part is that part's error
    assert m(ctypes.byref(pf(cu_seqlens_q=None)), ctypes.byref(dec(B=0)), None, *args, None, 0,
             None) == 1
    assert b"prefill part" in lib.pa_last_error()
    assert m(ctypes.byref(pf(B=0)), ctypes.byref(dec(out=None)), None, *args, None, 0, None) == 1
    assert b"decode part" in lib.pa_last_error()
    assert m(ctypes.byref(pf(B=-1)), ctypes.byref(dec()), None, *args, None, 0, None) == 2
    assert m(ctypes.byref(pf(B=0)), ctypes.byref(dec(max_seq_len=-5)), None, *args, None, 0,
             None) == 2
    assert m(ctypes.byref(pf()), ctypes.byref(dec()), None, FAKE, FAKE, P, ps, Hq, Hkv, 96, 0.1,
             None, 0, None) == 3
    # workspace: the prefill's parts for 256-row tiles, then the decode's partials
    need_pf = lib.paged_attn_prefill_workspace_bytes(2, 1200, 600, Hq, D, 3)
    need_dec = lib.paged_attn_decode_workspace_bytes(3, Hq, Hkv, D, 120, 2)
    assert need_pf > 0 and need_dec > 0
    assert w(ctypes.byref(pf()), ctypes.byref(dec()), None, Hq, Hkv, D) == need_pf + need_dec
    assert w(ctypes.byref(pf(B=0)), ctypes.byref(dec()), None, Hq, Hkv, D) == need_dec
    assert w(ctypes.byref(pf()), ctypes.byref(dec(B=0)), None, Hq, Hkv, D) == need_pf
    assert w(ctypes.byref(pf(num_splits=1)), ctypes.byref(dec(num_splits=1)), None, Hq, Hkv,
             D) == 0
    # the decode part's own count (num_splits <= 0): the decode's count (1 for 3 rows of
    # 120 keys) times the waves its launch would give each item (4 for 6 items), at most
    # one 32-key chunk per split
    assert lib.paged_attn_decode_num_splits(3, Hkv, 120) == 1
    assert w(ctypes.byref(pf(B=0)), ctypes.byref(dec(num_splits=0)), None, Hq, Hkv, D) == \
        lib.paged_attn_decode_workspace_bytes(3, Hq, Hkv, D, 120, 4)
    assert w(ctypes.byref(pf(B=0)), ctypes.byref(dec(num_splits=0, max_seq_len=70)), None, Hq,
             Hkv, D) == lib.paged_attn_decode_workspace_bytes(3, Hq, Hkv, D, 70, 3)
    assert w(None, ctypes.byref(dec()), None, Hq, Hkv, D) == 0
    # short prefill runs still take 256-row tiles, and the library's part count is
    # resolved for them: 4 x 32 x 2 tiles fill the 256 slots (one part), where the
    # prefill alone would take 128-row tiles, 384 of 512 slots, and two parts
    short = pf(B=4, max_q_len=300, num_splits=0)
    assert w(ctypes.byref(short), ctypes.byref(dec(B=0)), None, 32, Hkv, D) == 0
    assert lib.paged_attn_prefill_workspace_bytes(4, 1200, 300, 32, D, 0) > 0
    # a decode alone spreads over every CU: 32 rows of 8,192 keys at Hkv 4 take the
    # decode's 2 splits x 2 waves = 4 beside a prefill whose work-groups fill the chip
    # (4 x 4096 causal rows, Hq 28: 28 x 4 x 16 work-groups), but 16 alone (8 items per
    # work-group, 256 work-groups)
    big = dec(B=32, max_seq_len=8192, num_splits=0)
    c2 = lambda s: lib.paged_attn_decode_workspace_bytes(32, 28, 4, D, 8192, s)
    assert w(ctypes.byref(pf(B=0)), ctypes.byref(big), None, 28, 4, D) == c2(16)
    full = pf(B=4, Tq=16384, max_q_len=4096, num_splits=1)
    assert w(ctypes.byref(full), ctypes.byref(big), None, 28, 4, D) == c2(4)
    # a small prefill (2 x 300 rows, Hq 28: 112 work-groups) leaves 144 CUs: 9 splits
    small = pf(B=2, Tq=600, max_q_len=300, num_splits=1)
    assert w(ctypes.byref(small), ctypes.byref(big), None, 28, 4, D) == c2(9)
    # FP8 pools: the decode's own count for FP8 (1) times the waves the FP8 decode would
    # take (4), and the scales are checked as the separate entry points check them
    f8 = _lib.MixedFp8(0.5, 0.25, None, None)
    assert w(ctypes.byref(pf(B=0)), ctypes.byref(dec(num_splits=0)), ctypes.byref(f8), Hq,
             Hkv, D) == lib.paged_attn_decode_workspace_bytes(3, Hq, Hkv, D, 120, 4)
    bad = _lib.MixedFp8(-1.0, 0.25, None, None)
    assert m(ctypes.byref(pf(B=0)), ctypes.byref(dec()), ctypes.byref(bad), *args, None, 0,
             None) == 2
    half = _lib.MixedFp8(1.0, 1.0, FAKE, None)
    assert m(ctypes.byref(pf()), ctypes.byref(dec(B=0)), ctypes.byref(half), *args, None, 0,
             None) == 1
    for ws_bytes in (0, need_pf, need_pf + need_dec - 1):
        assert m(ctypes.byref(pf()), ctypes.byref(dec()), None, *args,
                 FAKE if ws_bytes else None, ws_bytes, None) == 5
        assert b"workspace" in lib.pa_last_error()
