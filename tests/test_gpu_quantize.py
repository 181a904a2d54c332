"""GPU parity of fp8attn_quantize against the CPU quantizer: E4M3 codes, per-head
scales and per-(segment, head, channel) K means must match bit for bit.

Q's scale follows the product's rule (amax/448 rounded up to a power-of-two
score factor, ``oracle.quantize.q_scale_pow2``); K and V use amax/448.

Quantization is independent across heads (every scale and mean is per head), so
at the full workload sizes the oracle is run on a seeded sample of heads over
all tokens; the small cases compare every head.
"""
import numpy as np
import pytest
import torch

import fp8_flash_attention_amd as fa
from oracle import quantize as Qz
from workloads import WORKLOADS, generate, make_workload
from tests.gpu_helpers import log, read_codes

pytestmark = pytest.mark.gpu


def _run_quantize(w, poison=False):
    q, k, v = generate(w, device="cuda")
    plan = fa.Plan(w.tokens, w.heads, w.cu_seqlens, w.softmax_scale, device=0)
    ws = plan.new_workspace()
    if poison:
        ws.fill_(0xFF)
    log(f"quantize {w.name} T={w.tokens} H={w.heads} cu={w.cu_seqlens[:8]} layout={w.layout}")
    fa.quantize(plan, q, k, v, ws)
    torch.cuda.synchronize()
    return plan, ws, (q.cpu(), k.cpu(), v.cpu())


def _check(w, heads, poison=False):
    plan, ws, (q, k, v) = _run_quantize(w, poison)
    got = read_codes(plan, ws, heads)
    hs = list(heads) if heads is not None else list(range(w.heads))
    exp = Qz.quantize(q[:, hs], k[:, hs], v[:, hs], w.cu_seqlens, w.softmax_scale)
    for name in ("q_codes", "k_codes", "v_codes"):
        a, b = got[name], exp[name]
        bad = np.argwhere(a != b)
        assert bad.size == 0, f"{name}: {len(bad)} code mismatches, first at {bad[0]}: gpu={a[tuple(bad[0])]:#x} " \
                              f"cpu={b[tuple(bad[0])]:#x}"
    assert np.array_equal(got["scales"][:, hs].view(np.uint32), exp["scales"].view(np.uint32))
    assert np.array_equal(got["mu"][:, hs].view(np.uint32), exp["mu"].view(np.uint32))
    for name, pad in got["pads"].items():
        assert not pad.size or not pad.any(), f"{name} padding bytes not zero"


@pytest.mark.parametrize("name", ["s256_h2", "s4096_h56"])
def test_codes_bit_exact_small(name):
    _check(WORKLOADS[name], None)


@pytest.mark.parametrize("name", ["s20440_h56_strided", "s30272_h56_koffset", "varlen_30272_h56"])
def test_codes_bit_exact_full_size_sampled_heads(name):
    _check(WORKLOADS[name], [0, 23, 55])


@pytest.mark.parametrize("cu", [
    [0, 1, 1, 64, 65, 200, 200, 457],       # empty, length-1, sub-tile and ragged segments
    [0, 0, 300],                             # leading empty segment
    [0, 256, 512, 513],                      # exact chunk boundaries then a single token
    [0, 1052],                               # regression lengths
    [0, 5980],
])
def test_codes_edge_segments(cu):
    w = make_workload("edge", cu[-1], 3, cu, seed=77, k_offset_var=2.0)
    _check(w, None)


def test_fused_qkv_strided_views():
    w = make_workload("fused", 700, 4, [0, 300, 700], seed=78, layout="fused")
    q, _, _ = generate(w)
    assert q.stride(0) == 3 * 4 * 128 and not q.is_contiguous()
    _check(w, None)


def test_poisoned_workspace_leaves_no_nan_byte():
    # every byte the pack pass owns is written, even inside a 0xFF-filled workspace
    w = make_workload("poison", 457, 3, [0, 1, 1, 64, 65, 200, 200, 457], seed=79)
    plan, ws, _ = _run_quantize(w, poison=True)
    for region in (0, 1, 2):
        codes = plan.region(ws, region).cpu().numpy()
        assert not np.any((codes & 0x7F) == 0x7F), f"region {region} holds a NaN code"
    _check(w, None, poison=True)


def test_zero_head_scale():
    # all-zero K and V heads get scale 1; an all-zero Q head gets 1 rounded up
    # to a power-of-two score factor; every code of such a head is zero
    w = make_workload("zeros", 300, 2, [0, 300], seed=80)
    q, k, v = generate(w, device="cuda")
    q[:, 1] = 0
    k[:, 1] = 3.0          # constant K: centred to exactly zero
    v[:, 0] = 0
    plan = fa.Plan(w.tokens, w.heads, w.cu_seqlens, device=0)
    ws = plan.new_workspace()
    log("quantize zero heads")
    fa.quantize(plan, q, k, v, ws)
    torch.cuda.synchronize()
    sc = plan.region(ws, 3).cpu().numpy()
    assert sc[1, 1] == 1.0 and sc[2, 0] == 1.0 and 1.0 <= sc[0, 1] < 2.0
    exp = Qz.quantize(q.cpu(), k.cpu(), v.cpu(), w.cu_seqlens, w.softmax_scale)
    assert np.array_equal(sc.view(np.uint32), exp["scales"].view(np.uint32))
    got = read_codes(plan, ws)
    assert not got["q_codes"][:, 1].any() and not got["v_codes"][:, 0].any()
    for name in ("q_codes", "k_codes", "v_codes"):
        assert np.array_equal(got[name], exp[name])


def test_empty_input():
    plan = fa.Plan(0, 2, [0, 0], device=0)
    ws = plan.new_workspace()
    x = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    log("quantize empty")
    fa.quantize(plan, x, x, x, ws)
    out = fa.forward(plan, ws)
    torch.cuda.synchronize()
    assert out.shape == (0, 2, 128)


def _segment_scaled_inputs():
    # segments of very different magnitudes, an empty segment and a 1-token one
    cu = [0, 200, 200, 513, 699, 700]
    w = make_workload("segscale", 700, 3, cu, seed=111)
    q, k, v = generate(w)
    q[200:513] *= 8
    k[0:200] += 2
    v[513:699] *= 0.25
    v[699:] *= 40
    return w, q, k, v


def test_segment_scales_codes_bit_exact():
    w, q, k, v = _segment_scaled_inputs()
    plan = fa.Plan(w.tokens, w.heads, w.cu_seqlens, w.softmax_scale, device=0, segment_scales=True)
    ws = plan.new_workspace()
    ws.fill_(0xFF)
    log(f"quantize with per-segment scales cu={w.cu_seqlens}")
    fa.quantize(plan, q.cuda(), k.cuda(), v.cuda(), ws)
    torch.cuda.synchronize()
    got = read_codes(plan, ws)
    exp = Qz.quantize_segments(q, k, v, w.cu_seqlens, w.softmax_scale)
    for name in ("q_codes", "k_codes", "v_codes"):
        assert np.array_equal(got[name], exp[name]), name
    assert got["scales"].shape == (3, len(w.cu_seqlens) - 1, w.heads)
    assert np.array_equal(got["scales"].view(np.uint32), exp["scales"].view(np.uint32))
    assert np.array_equal(got["mu"].view(np.uint32), exp["mu"].view(np.uint32))
    for name, pad in got["pads"].items():
        assert not pad.size or not pad.any(), f"{name} padding bytes not zero"
    # per-head scales over the whole call differ on these inputs
    base = Qz.quantize(q, k, v, w.cu_seqlens, w.softmax_scale)
    assert not np.array_equal(base["v_codes"], exp["v_codes"])
