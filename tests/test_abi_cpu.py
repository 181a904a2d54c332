"""CPU checks of the C-ABI library: it loads, exports every declared symbol,
validates arguments, and builds the documented schedule.  No GPU compute.

Host-only plans (device = -1) exercise the planner without a device.
"""
import ctypes
import os
import re

import pytest

from fp8_flash_attention_amd import _lib
import fp8_flash_attention_amd as fa
from workloads import WORKLOADS

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")


def _declared():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            txt = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, h)).read(), flags=re.S)
            names |= set(re.findall(r"\b(fp8attn_[a-z_]+)\s*\(", txt))
    return sorted(names)


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 9
    L = _lib.lib()
    for n in names:
        assert hasattr(L, n), n
        assert n in _lib.SIGNATURES, f"{n} has no ctypes signature"


def _plan(tokens, heads, cu, scale=0.088, device=-1):
    L = _lib.lib()
    h = ctypes.c_void_p()
    arr = (ctypes.c_int32 * len(cu))(*cu)
    st = L.fp8attn_plan(ctypes.byref(h), tokens, heads, arr, len(cu) - 1, ctypes.c_float(scale), device)
    return st, h


@pytest.mark.parametrize("tokens,heads,cu,scale,msg", [
    (10, 2, [1, 10], 0.1, "cu_seqlens[0]"),
    (10, 2, [0, 6, 5, 10], 0.1, "non-decreasing"),
    (10, 2, [0, 9], 0.1, "equal tokens"),
    (10, 0, [0, 10], 0.1, "heads"),
    (-1, 2, [0, -1], 0.1, "tokens"),
    (10, 2, [0, 10], 0.0, "softmax_scale"),
    (10, 2, [0, 10], float("nan"), "softmax_scale"),
    (10, 2, [0, 10], float("inf"), "softmax_scale"),
    (10, 2, [0, 10], -1.0, "softmax_scale"),
])
def test_plan_rejects_bad_arguments(tokens, heads, cu, scale, msg):
    st, h = _plan(tokens, heads, cu, scale)
    assert st == _lib.EINVAL
    assert h.value is None
    assert msg in _lib.lib().fp8attn_last_error().decode()


def test_plan_null_arguments():
    L = _lib.lib()
    h = ctypes.c_void_p()
    assert L.fp8attn_plan(None, 1, 1, (ctypes.c_int32 * 2)(0, 1), 1, ctypes.c_float(1.0), -1) == _lib.EINVAL
    assert L.fp8attn_plan(ctypes.byref(h), 1, 1, None, 1, ctypes.c_float(1.0), -1) == _lib.EINVAL
    assert L.fp8attn_plan(ctypes.byref(h), 1, 1, (ctypes.c_int32 * 2)(0, 1), 0, ctypes.c_float(1.0), -1) == _lib.EINVAL
    assert L.fp8attn_workspace_bytes(None) == 0
    assert L.fp8attn_plan_destroy(None) == _lib.OK


def test_host_only_plan_cannot_run():
    p = fa.Plan(256, 2, [0, 256], device=-1)
    L = _lib.lib()
    s = _lib.i64_array([256, 128])
    st = L.fp8attn_quantize(p.handle, ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), s, s, s,
                            ctypes.c_void_p(256), p.workspace_bytes, None)
    assert st == _lib.EINVAL and "host-only" in L.fp8attn_last_error().decode()
    st = L.fp8attn_forward(p.handle, ctypes.c_void_p(256), p.workspace_bytes, ctypes.c_void_p(16), s, None, None)
    assert st == _lib.EINVAL


def _expected_items(cu, heads, bm):
    segs = [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]
    return heads * sum((L + bm - 1) // bm for L in segs)


CUS_PER_XCD = 32        # host-only plans assume 256 CUs over 8 XCDs


def _wg_per_cu(bm):
    return 1 if bm == 256 else 2     # attention workgroups resident per CU


def _split(w):
    return w & 15, (w >> 4) & 15, w >> 8      # piece index, piece count, first partial slot


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_schedule_for_each_workload(name):
    w = WORKLOADS[name]
    p = fa.Plan(w.tokens, w.heads, w.cu_seqlens, device=-1)
    info = p.info()
    assert info["tokens"] == w.tokens and info["heads"] == w.heads
    assert info["num_segments"] == len(w.cu_seqlens) - 1
    bm = info["query_tile"]
    assert bm in (128, 256) and info["key_tile"] == 64
    segs = w.segments
    assert info["workspace_rows"] == sum((L + 127) // 128 * 128 for L in segs) + 128
    assert info["stat_chunks"] == sum((L + 255) // 256 for L in segs)
    items = p.work_items()
    assert len(items) % 8 == 0
    real = [it for it in items if it[0] >= 0]
    assert len(real) == info["work_items"]
    # every (segment, query tile, head) appears exactly once, whole or as a complete
    # set of key pieces; empty segments never appear
    want = {(s, q0, h) for h in range(w.heads) for s, L in enumerate(segs) for q0 in range(0, L, bm)}
    whole = [(s, q0, h) for s, q0, h, sp in real if sp == 0]
    pieces = {}
    for s, q0, h, sp in real:
        if sp:
            i, n, base = _split(sp)
            pieces.setdefault((s, q0, h), []).append((i, n, base))
    assert len(set(whole)) == len(whole) and not set(whole) & set(pieces)
    assert set(whole) | set(pieces) == want
    assert len(whole) + len(pieces) == _expected_items(w.cu_seqlens, w.heads, bm)
    slots = []
    for (s, q0, h), ps in pieces.items():
        n, base = ps[0][1], ps[0][2]
        assert 2 <= n <= 8 and sorted(i for i, _, _ in ps) == list(range(n))
        assert all(pn == n and pb == base for _, pn, pb in ps)
        nkt = (segs[s] + 63) // 64
        bounds = [nkt * i // n for i in range(n + 1)]
        assert bounds[0] == 0 and bounds[-1] == nkt
        assert min(b - a for a, b in zip(bounds, bounds[1:])) >= 8
        slots += [base + i for i in range(n)]
    assert sorted(slots) == list(range(len(slots)))
    # XCD interleave: workgroup i belongs to XCD i % 8 and each XCD walks a contiguous
    # run of the head-major list, longest items first; split pieces only at the end,
    # filling what would otherwise be a last round at most half full
    per = len(items) // 8
    for x in range(8):
        run = [items[x + 8 * j] for j in range(per)]
        run = [it for it in run if it[0] >= 0]
        first_piece = next((j for j, it in enumerate(run) if it[3]), len(run))
        assert all(it[3] for it in run[first_piece:])
        head = run[:first_piece]
        sizes = [(segs[it[0]] + 63) // 64 for it in head]
        assert sizes == sorted(sizes, reverse=True)
        for size in set(sizes):
            hs = [it[2] for it in head if (segs[it[0]] + 63) // 64 == size]
            assert hs == sorted(hs)


def _expected_pieces(items_in_part, tiles, bm):
    """The documented split rule for one XCD's part of equal-length items."""
    slots = _wg_per_cu(bm) * CUS_PER_XCD
    r = items_in_part % slots
    if r == 0 or 2 * r > CUS_PER_XCD:
        return 0, 1
    return r, min(8, CUS_PER_XCD // r, tiles // 8)


@pytest.mark.parametrize("name", ["s30272_h7_shard", "s4096_h56", "s30272_h56_koffset", "s20440_h56_strided"])
def test_split_fills_the_last_round(name):
    # single-segment workloads: every XCD part holds equal items; the items of a last
    # round that would leave at least half the XCD's CUs idle are split into as many
    # key pieces as fit one per CU (at most 8, at least 8 key tiles each)
    w = WORKLOADS[name]
    p = fa.Plan(w.tokens, w.heads, w.cu_seqlens, device=-1)
    bm = p.info()["query_tile"]
    tiles = (w.tokens + 63) // 64
    n_items = w.heads * ((w.tokens + bm - 1) // bm)
    per = (n_items + 7) // 8
    want = []
    for x in range(8):
        in_part = max(0, min(per, n_items - x * per))
        r, n = _expected_pieces(in_part, tiles, bm)
        want.append((r, n if r and n >= 2 else 1))
    items = p.work_items()
    for x in range(8):
        run = [it for it in items[x::8] if it[0] >= 0]
        pieces = [it for it in run if it[3]]
        r, n = want[x]
        if n < 2:
            assert not pieces
        else:
            assert len(pieces) == r * n and {_split(it[3])[1] for it in pieces} == {n}


@pytest.mark.parametrize("name,query_tile,split_items,pieces_each", [
    ("s256_h2", 128, 0, 0),               # a few rounds deep: 128-query items
    ("s4096_h56", 128, 0, 0),             # 3.5 rounds of 256-query items: 128-query items, 7 full rounds
    ("s20440_h56_strided", 256, 128, 2),  # last round of exactly half the CUs of each XCD: split
    ("s30272_h56_koffset", 256, 8, 8),    # one item left per XCD: eight pieces
    ("varlen_30272_h56", 256, 0, 0),
])
def test_graded_workloads_split_counts(name, query_tile, split_items, pieces_each):
    # the query tile and split schedule of each graded workload on a 256-CU
    # device, as stated in the design notes
    w = WORKLOADS[name]
    p = fa.Plan(w.tokens, w.heads, w.cu_seqlens, device=-1)
    assert p.info()["query_tile"] == query_tile
    pieces = [it for it in p.work_items() if it[0] >= 0 and it[3]]
    items = {(it[0], it[1], it[2]) for it in pieces}
    assert len(items) == split_items
    assert len(pieces) == split_items * pieces_each == p.info()["partial_slots"]
    assert all(_split(it[3])[1] == pieces_each for it in pieces)


def test_split_small_and_short_cases():
    # few items: as many pieces as fit one per CU, at least 8 key tiles each
    p = fa.Plan(3000, 1, [0, 3000], device=-1)
    ns = {_split(it[3])[1] for it in p.work_items() if it[0] >= 0}
    assert ns == {5}      # <= 2 items per XCD -> min(8, 32 // 2, 47 // 8) = 5
    # segments shorter than 16 key tiles are never split
    p = fa.Plan(300, 8, [0, 300], device=-1)
    assert not any(it[3] for it in p.work_items())


def test_varlen_schedule_longest_segment_first():
    w = WORKLOADS["varlen_30272_h56"]
    p = fa.Plan(w.tokens, w.heads, w.cu_seqlens, device=-1)
    items = p.work_items()
    per = len(items) // 8
    lin = [items[(j % per) * 8 + j // per] for j in range(len(items))]
    head0 = [it for it in lin if it[0] >= 0 and it[2] == 0]
    segs = [it[0] for it in head0]
    # segment lengths 15104, 15104, 0, 63, 1: the two long ones first, then 63, then 1
    n = (15104 + p.info()["query_tile"] - 1) // p.info()["query_tile"]
    assert segs[:n] == [0] * n and segs[n:2 * n] == [1] * n and segs[2 * n:] == [3, 4]


def test_plan_rejects_rows_beyond_32bit_code_offsets():
    # one head's code rows are addressed with 32-bit byte offsets: rows * 128 < 2^31
    ok = 16_777_087 - 127              # padded to a multiple of 128, plus 128 guard rows
    st, h = _plan(ok, 1, [0, ok])
    assert st == _lib.OK
    _lib.lib().fp8attn_plan_destroy(h)
    big = 16_777_216
    st, h = _plan(big, 1, [0, big])
    assert st == _lib.EUNSUPPORTED and h.value is None
    assert "32-bit" in _lib.lib().fp8attn_last_error().decode()
    # the pack grid holds (rows / 64) x heads blocks in one dimension; heads in another
    st, h = _plan(4_000_000, 40_000, [0, 4_000_000])
    assert st == _lib.EUNSUPPORTED and h.value is None
    st, h = _plan(64, 65536, [0, 64])
    assert st == _lib.EUNSUPPORTED and h.value is None
    st, h = _plan(64, 65535, [0, 64])
    assert st == _lib.OK
    _lib.lib().fp8attn_plan_destroy(h)


def test_plan_ex_flags_and_segment_scale_layout():
    L = _lib.lib()
    cu = (ctypes.c_int32 * 4)(0, 100, 100, 300)
    h = ctypes.c_void_p()
    assert L.fp8attn_plan_ex(ctypes.byref(h), 300, 2, cu, 3, ctypes.c_float(0.088), -1, 64) == _lib.EINVAL
    assert "flags" in L.fp8attn_last_error().decode()
    assert L.fp8attn_plan_ex(ctypes.byref(h), 300, 2, cu, 3, ctypes.c_float(0.088), -1,
                             _lib.PLAN_EXACT_PROBS | _lib.PLAN_MXFP4) == _lib.EINVAL
    assert L.fp8attn_plan_ex(ctypes.byref(h), 300, 2, cu, 3, ctypes.c_float(0.088), -1, _lib.PLAN_EXACT_PROBS) == 0
    L.fp8attn_plan_destroy(h)
    base = fa.Plan(300, 2, [0, 100, 100, 300], device=-1)
    seg = fa.Plan(300, 2, [0, 100, 100, 300], device=-1, segment_scales=True)
    assert base.info()["segment_scales"] == 0 and seg.info()["segment_scales"] == 1
    ptr = ctypes.c_void_p()
    dims = (ctypes.c_int64 * 3)()
    assert L.fp8attn_workspace_region(base.handle, ctypes.c_void_p(1 << 20), _lib.REGION_SCALES,
                                      ctypes.byref(ptr), dims) == 0
    assert tuple(dims) == (3, 1, 2)
    assert L.fp8attn_workspace_region(seg.handle, ctypes.c_void_p(1 << 20), _lib.REGION_SCALES,
                                      ctypes.byref(ptr), dims) == 0
    assert tuple(dims) == (3, 3, 2)                 # one set per segment, the empty one included
    assert seg.workspace_bytes >= base.workspace_bytes
    # the work schedule does not depend on the scale mode
    assert seg.work_items() == base.work_items()


def test_empty_input_plan():
    p = fa.Plan(0, 3, [0, 0], device=-1)
    info = p.info()
    assert info["work_items"] == 0 and info["stat_chunks"] == 0
    assert p.workspace_bytes > 0


def test_workspace_region_host_plan():
    p = fa.Plan(300, 2, [0, 100, 300], device=-1)
    L = _lib.lib()
    ptr = ctypes.c_void_p()
    dims = (ctypes.c_int64 * 3)()
    base = 1 << 20
    assert L.fp8attn_workspace_region(p.handle, ctypes.c_void_p(base), _lib.REGION_V, ctypes.byref(ptr), dims) == 0
    rows = 128 + 256 + 128
    assert tuple(dims) == (2, 128, rows)
    assert L.fp8attn_workspace_region(p.handle, ctypes.c_void_p(base), _lib.REGION_MU, ctypes.byref(ptr), dims) == 0
    assert tuple(dims) == (2, 2, 128)
    assert L.fp8attn_workspace_region(p.handle, ctypes.c_void_p(base), 99, ctypes.byref(ptr), dims) == _lib.EINVAL
    assert L.fp8attn_workspace_region(p.handle, ctypes.c_void_p(base), _lib.REGION_ROWMAP,
                                      ctypes.byref(ptr), dims) == _lib.EINVAL


def test_python_wrapper_rejects_unsupported():
    import torch
    with pytest.raises(fa.Fp8AttnError):                 # FP4 plans of 64 channels
        fa.Plan(256, 2, [0, 256], device=-1, fmt="mxfp4", head_dim=64)
    with pytest.raises(ValueError):                      # head_dim other than 128
        fa._strides(torch.zeros((4, 2, 64), dtype=torch.bfloat16), "q")
    with pytest.raises(TypeError):                       # non-BF16 input
        fa._strides(torch.zeros((4, 2, 128), dtype=torch.float16), "q")


def test_mxfp4_plan_flags_layout_and_schedule():
    L = _lib.lib()
    cu = (ctypes.c_int32 * 4)(0, 100, 100, 300)
    h = ctypes.c_void_p()
    # E4M3 Q centring takes any head size; FP4 takes no per-segment scales
    for extra in (_lib.PLAN_HEAD_DIM_64, _lib.plan_head_dim(40), 0):
        assert L.fp8attn_plan_ex(ctypes.byref(h), 300, 2, cu, 3, ctypes.c_float(0.088), -1,
                                 _lib.PLAN_Q_CENTRE | extra) == _lib.OK
        L.fp8attn_plan_destroy(h)
        h = ctypes.c_void_p()
    assert L.fp8attn_plan_ex(ctypes.byref(h), 300, 2, cu, 3, ctypes.c_float(0.088), -1,
                             _lib.PLAN_MXFP4 | _lib.PLAN_SEGMENT_SCALES) == _lib.EINVAL
    assert h.value is None
    e4 = fa.Plan(300, 2, [0, 100, 100, 300], device=-1)
    mx = fa.Plan(300, 2, [0, 100, 100, 300], device=-1, fmt="mxfp4", q_centre=True)
    info = mx.info()
    assert info["mxfp4"] == 1 and info["q_centre"] == 1 and e4.info()["mxfp4"] == 0
    assert info["partial_slots"] == 0
    rows = info["workspace_rows"]
    assert rows == 128 + 256 + 128
    ptr = ctypes.c_void_p()
    dims = (ctypes.c_int64 * 3)()
    base = 1 << 20
    want = {_lib.REGION_Q: (2, rows, 64), _lib.REGION_K: (2, rows, 64), _lib.REGION_V: (2, rows // 64, 4096),
            _lib.REGION_Q_BSCALES: (2, rows, 4), _lib.REGION_K_BSCALES: (2, rows, 4),
            _lib.REGION_V_BSCALES: (2, rows // 64, 256), _lib.REGION_QM_CODES: (2, rows // 128, 64),
            _lib.REGION_QM_SCALES: (2, rows // 128, 4), _lib.REGION_MU: (3, 2, 128)}
    offs = []
    for which, shape in want.items():
        assert L.fp8attn_workspace_region(mx.handle, ctypes.c_void_p(base), which, ctypes.byref(ptr), dims) == 0
        assert tuple(dims) == shape, which
        offs.append((ptr.value - base, shape[0] * shape[1] * shape[2] * (4 if which == _lib.REGION_MU else 1)))
    offs.sort()
    for (o0, n0), (o1, _) in zip(offs, offs[1:]):
        assert o0 + n0 <= o1                          # regions do not overlap
    assert offs[-1][0] + offs[-1][1] <= mx.workspace_bytes
    assert L.fp8attn_workspace_region(mx.handle, ctypes.c_void_p(base), _lib.REGION_SCALES,
                                      ctypes.byref(ptr), dims) == _lib.EINVAL
    # E4M3 regions are not reported for FP4 planes and vice versa
    assert L.fp8attn_workspace_region(e4.handle, ctypes.c_void_p(base), _lib.REGION_Q_BSCALES,
                                      ctypes.byref(ptr), dims) == _lib.EINVAL
    assert mx.workspace_bytes < e4.workspace_bytes


def test_mxfp4_plan_schedule_and_splits():
    """The graded schedules have no split items as FP4 (every (segment,
    128-query tile, head) once); a schedule that leaves a short last round is
    split along the keys as for E4M3 plans, and its workspace holds the
    partial regions."""
    for cu in ([0, 4096], [0, 15104, 30208, 30208, 30271, 30272], [0, 2048, 2100]):
        T = cu[-1]
        e4 = fa.Plan(T, 56, cu, device=-1)
        mx = fa.Plan(T, 56, cu, device=-1, fmt="mxfp4")
        assert mx.info()["query_tile"] == 128 and e4.info()["query_tile"] in (128, 256)
        items = mx.work_items()
        assert all(it[3] == 0 for it in items)
        real = [it for it in items if it[0] >= 0]
        want = {(s, q0, h, 0) for s in range(len(cu) - 1) for h in range(56)
                for q0 in range(0, cu[s + 1] - cu[s], 128)}
        assert len(real) == len(want) and set(real) == want
        assert mx.info()["work_items"] == len(real)
    # 2048 tokens x 4 heads: 64 items, 8 per XCD, a last round of 8 items
    # for 32 compute units: each item in four pieces of 8 key tiles
    cu = [0, 2048]
    mx = fa.Plan(2048, 4, cu, device=-1, fmt="mxfp4")
    items = [it for it in mx.work_items() if it[0] >= 0]
    assert all(it[3] != 0 for it in items)
    assert {(it[3] >> 4) & 15 for it in items} == {4}
    assert mx.info()["partial_slots"] == 64 * 4
    pieces = {}
    for s, q0, h, w in items:
        pieces.setdefault((s, q0, h, w >> 8), []).append(w & 15)
    assert len(pieces) == 64 and all(sorted(v) == [0, 1, 2, 3] for v in pieces.values())
    nosplit = fa.Plan(4096, 56, [0, 4096], device=-1, fmt="mxfp4")
    assert nosplit.info()["partial_slots"] == 0
    # the partial slots (256 rows of 128 floats, plus two floats a row) are in the workspace
    assert mx.workspace_bytes >= 256 * 256 * (128 + 2) * 4


def test_causal_plan_schedule():
    """Causal items attend to the key tiles up to their last query; no splits;
    per XCD part, longer items first."""
    cu = [0, 4096, 4096, 4500]
    p = fa.Plan(4500, 8, cu, device=-1, causal=True)
    assert p.info()["causal"] == 1 and p.info()["partial_slots"] == 0
    items = [it for it in p.work_items() if it[0] >= 0]
    assert all(it[3] == 0 for it in items)
    segs = {0: 4096, 2: 404}
    want = {(s, q0, h) for s, L in segs.items() for h in range(8) for q0 in range(0, L, 256)}
    assert {(s, q, h) for s, q, h, _ in items} == want
    assert p.info()["work_items"] == len(items)
    # causal FP4 plans: 128-query items, no splits, every (segment, tile, head) once
    mx = fa.Plan(4500, 8, cu, device=-1, causal=True, fmt="mxfp4", q_centre=True)
    assert mx.info()["causal"] == 1 and mx.info()["partial_slots"] == 0 and mx.info()["query_tile"] == 128
    items = [it for it in mx.work_items() if it[0] >= 0]
    assert all(it[3] == 0 for it in items)
    want = {(s, q0, h) for s, L in segs.items() for h in range(8) for q0 in range(0, L, 128)}
    assert len(items) == len(want) and {(s, q, h) for s, q, h, _ in items} == want


def test_batched_wrapper_rejects_cu_seqlens():
    import torch
    q = torch.zeros((2, 4, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.attention(q, q, q, cu_seqlens=[0, 4, 8])


def test_causal_parts_balanced_and_local():
    """Causal schedule: the XCD parts (item j*8 + x of the launch order goes to
    XCD x) carry equal work up to one item, and an XCD's first round of
    workgroups stays on a few heads."""
    T, H = 30272, 56
    p = fa.Plan(T, H, [0, T], device=-1, causal=True)
    items = p.work_items()
    tiles = lambda it: (min(T, it[1] + 256) + 63) // 64
    work = []
    for x in range(8):
        part = [it for it in items[x::8] if it[0] >= 0]
        work.append(sum(tiles(it) for it in part))
        first_round = part[:32]
        assert len({it[2] for it in first_round}) <= 4          # heads in flight on the XCD
        assert tiles(first_round[0]) == max(tiles(it) for it in part[:len(first_round)])
    assert max(work) - min(work) <= (T + 63) // 64


def test_head_dim_64_plan_layout():
    L = _lib.lib()
    h = ctypes.c_void_p()
    arr = (ctypes.c_int32 * 3)(0, 100, 300)
    assert L.fp8attn_plan_ex(ctypes.byref(h), 300, 2, arr, 2, ctypes.c_float(0.125), -1,
                             _lib.PLAN_HEAD_DIM_64 | _lib.PLAN_MXFP4) == _lib.EINVAL
    p = fa.Plan(300, 2, [0, 100, 300], device=-1, head_dim=64)
    p128 = fa.Plan(300, 2, [0, 100, 300], device=-1)
    assert p.info()["head_dim"] == 64 and p128.info()["head_dim"] == 128
    assert p.softmax_scale == pytest.approx(0.125)
    rows = p.info()["workspace_rows"]
    ptr = ctypes.c_void_p()
    dims = (ctypes.c_int64 * 3)()
    for which, shape in ((_lib.REGION_Q, (2, rows, 64)), (_lib.REGION_V, (2, 64, rows)), (_lib.REGION_MU, (2, 2, 64))):
        assert L.fp8attn_workspace_region(p.handle, ctypes.c_void_p(1 << 20), which, ctypes.byref(ptr), dims) == 0
        assert tuple(dims) == shape
    assert p.workspace_bytes < p128.workspace_bytes
    # 64-channel plans always run 256-query items (the 128-channel plan of this
    # shallow grid runs 128-query ones)
    assert p.info()["query_tile"] == 256 and p128.info()["query_tile"] == 128
    real = {it for it in p.work_items() if it[0] >= 0}
    assert real == {(s, q0, h, 0) for h in range(2) for s, (a, b) in enumerate([(0, 100), (100, 300)])
                    for q0 in range(0, b - a, 256)}
    for bad in (0, 4, 100, 136, 256):
        with pytest.raises(ValueError):
            fa.Plan(300, 2, [0, 300], device=-1, head_dim=bad)


@pytest.mark.parametrize("d,dk", [(8, 64), (32, 64), (64, 64), (72, 128), (96, 128), (120, 128), (128, 128)])
def test_head_dim_flag_and_kernel_width(d, dk):
    """FP8ATTN_PLAN_HEAD_DIM(d): q, k, v and out have d channels; the code
    regions and K means have the kernel width (64 or 128)."""
    L = _lib.lib()
    p = fa.Plan(300, 2, [0, 100, 300], device=-1, head_dim=d)
    assert p.info()["head_dim"] == d and p.softmax_scale == pytest.approx(d ** -0.5)
    rows = p.info()["workspace_rows"]
    ptr = ctypes.c_void_p()
    dims = (ctypes.c_int64 * 3)()
    for which, shape in ((_lib.REGION_Q, (2, rows, dk)), (_lib.REGION_V, (2, dk, rows)), (_lib.REGION_MU, (2, 2, dk))):
        assert L.fp8attn_workspace_region(p.handle, ctypes.c_void_p(1 << 20), which, ctypes.byref(ptr), dims) == 0
        assert tuple(dims) == shape
    same = fa.Plan(300, 2, [0, 100, 300], device=-1, head_dim=64 if dk == 64 else 128)
    assert p.workspace_bytes == same.workspace_bytes
    assert p.info()["query_tile"] == same.info()["query_tile"]


def test_head_dim_flag_errors():
    L = _lib.lib()
    h = ctypes.c_void_p()
    arr = (ctypes.c_int32 * 2)(0, 256)
    def plan(flags):
        return L.fp8attn_plan_ex(ctypes.byref(h), 256, 2, arr, 1, ctypes.c_float(0.125), -1, flags)
    assert plan(_lib.plan_head_dim(96) | _lib.PLAN_MXFP4) == _lib.EINVAL           # FP4: 128 only
    assert plan(_lib.plan_head_dim(96) | _lib.PLAN_HEAD_DIM_64) == _lib.EINVAL     # two different sizes
    assert plan(_lib.plan_head_dim(136)) == _lib.EINVAL                            # above 128
    assert plan(_lib.plan_head_dim(64) | _lib.PLAN_HEAD_DIM_64) == _lib.OK         # the same size twice
    L.fp8attn_plan_destroy(h)
    assert plan(_lib.plan_head_dim(40) | _lib.PLAN_CAUSAL | _lib.PLAN_SEGMENT_SCALES) == _lib.OK
    L.fp8attn_plan_destroy(h)


def test_quantize_noalloc_rejects_plans_beyond_its_static_buffer():
    # checked before anything else, so a host-only plan shows it without a GPU
    L = _lib.lib()
    big = fa.Plan(320_037, 56, [0, 320_037], device=-1)
    rc = L.fp8attn_quantize_noalloc(big.handle, None, None, None, None, None, None, None, 0, None)
    assert rc == _lib.EUNSUPPORTED and b"static buffer" in L.fp8attn_last_error()
    # a plan whose statistics fit gets past that check (and stops at the host-only one)
    small = fa.Plan(30272, 56, [0, 15104, 30208, 30208, 30271, 30272], device=-1)
    rc = L.fp8attn_quantize_noalloc(small.handle, None, None, None, None, None, None, None, 0, None)
    assert rc == _lib.EINVAL and b"host-only" in L.fp8attn_last_error()


def test_statistics_region_is_last():
    # fp8attn_quantize_noalloc and fp8attn_forward need only the bytes before it
    for flags in ({}, {"fmt": "mxfp4"}, {"segment_scales": True}, {"head_dim": 64}):
        p = fa.Plan(4096, 8, [0, 1000, 4096], device=-1, **flags)
        off = p.stats_offset()
        assert 0 < off < p.workspace_bytes and off % 256 == 0


def test_plan_cache_is_bounded_and_lru():
    # host-only plans: the cache keeps at most PLAN_CACHE_SIZE plans, evicts the least
    # recently used one and frees it
    fa.clear_plan_cache()
    n = fa.PLAN_CACHE_SIZE
    made = [fa.get_plan(100 + i, 2, [0, 100 + i], 0.1, -1) for i in range(n)]
    assert len(fa._PLANS) == n
    again = fa.get_plan(100, 2, [0, 100], 0.1, -1)          # a hit moves it to the back
    assert again is made[0]
    extra = [fa.get_plan(1000 + i, 2, [0, 1000 + i], 0.1, -1) for i in range(n + 3)]
    assert len(fa._PLANS) == n
    assert all(p.handle is None for p in made)              # evicted and destroyed
    assert all(p.handle is not None for p in extra[-n:])
    fa.clear_plan_cache()
    assert not fa._PLANS and all(p.handle is None for p in extra)


def test_varlen_entry_points_validate_arguments():
    import torch
    q = torch.zeros((64, 2, 128), dtype=torch.bfloat16)
    for bad in ([0, 64], torch.tensor([0, 64], dtype=torch.int64), torch.tensor([[0, 64]], dtype=torch.int32)):
        with pytest.raises(ValueError):
            fa.varlen_attention_fp8(q, q, q, bad)
    with pytest.raises(ValueError):                        # wrong head size
        z = torch.zeros((64, 2, 96), dtype=torch.bfloat16)
        fa.varlen_attention_mxfp4(z, z, z, torch.tensor([0, 64], dtype=torch.int32))
    with pytest.raises(ValueError):                        # host copy of another length
        fa.varlen_attention_fp8(q, q, q, torch.tensor([0, 64], dtype=torch.int32), cu_seqlens_host=[0, 32, 64])
    assert fa.workspace_bytes(0) == 0


def test_e4m3_q_centre_plan_layout_and_regions():
    """E4M3 plans with Q centring: block means [H][rows/128][128] and the
    mean-term table of sum over segments of (Lr/128) * Lr entries per head
    (Lr = the segment's rows rounded up to 128), both before the statistics;
    the Q block statistics inside them."""
    cu = [0, 100, 100, 300, 557]
    H = 3
    plain = fa.Plan(557, H, cu, device=-1)
    qc = fa.Plan(557, H, cu, device=-1, q_centre=True)
    assert qc.info()["q_centre"] == 1 and plain.info()["q_centre"] == 0
    rows = qc.info()["workspace_rows"]
    assert rows == 128 + 256 + 384 + 128
    lrs = [(b - a + 127) // 128 * 128 for a, b in zip(cu[:-1], cu[1:])]
    entries = sum((lr // 128) * lr for lr in lrs)
    assert entries == 128 + 2 * 256 + 3 * 384
    L = _lib.lib()
    base = 1 << 20
    ptr = ctypes.c_void_p()
    dims = (ctypes.c_int64 * 3)()
    assert L.fp8attn_workspace_region(qc.handle, ctypes.c_void_p(base), _lib.REGION_QMEAN, ctypes.byref(ptr),
                                      dims) == _lib.OK
    assert tuple(dims) == (H, rows // 128, 128)
    qmean_off = ptr.value - base
    assert L.fp8attn_workspace_region(qc.handle, ctypes.c_void_p(base), _lib.REGION_QM_TERM, ctypes.byref(ptr),
                                      dims) == _lib.OK
    assert tuple(dims) == (H, entries, 4)
    mt_off = ptr.value - base
    assert mt_off >= qmean_off + 4 * H * (rows // 128) * 128
    assert qc.stats_offset() >= mt_off + 4 * H * entries
    # the statistics grow by the blocks' centred amax partials (16 floats per block and head)
    grow = (qc.workspace_bytes - qc.stats_offset()) - (plain.workspace_bytes - plain.stats_offset())
    assert grow >= 4 * 16 * (rows // 128) * H
    for which in (_lib.REGION_QMEAN, _lib.REGION_QM_TERM):
        assert L.fp8attn_workspace_region(plain.handle, ctypes.c_void_p(base), which, ctypes.byref(ptr),
                                          dims) == _lib.EINVAL
    # the schedule is the one of the plain plan
    assert qc.work_items() == plain.work_items()


def test_e4m3_q_centre_rejects_segments_beyond_32_bit_table_offsets():
    L = _lib.lib()
    h = ctypes.c_void_p()
    for T, ok in ((262016, True), (262017, False)):
        cu = (ctypes.c_int32 * 2)(0, T)
        st = L.fp8attn_plan_ex(ctypes.byref(h), T, 1, cu, 1, ctypes.c_float(0.088), -1, _lib.PLAN_Q_CENTRE)
        assert st == (_lib.OK if ok else _lib.EUNSUPPORTED), (T, st)
        if ok:
            L.fp8attn_plan_destroy(h)
