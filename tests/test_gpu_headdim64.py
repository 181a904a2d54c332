"""GPU parity of head_dim-64 plans (FP8ATTN_PLAN_HEAD_DIM_64) against the CPU
oracle, with the bars of the 128-channel path: E4M3 codes, scales and K means
bit for bit; the output graded against the exact inputs (relative RMS <= 0.06,
|o - r| <= 0.1 + 0.1 |r|) and against the oracle on the dequantized operands
(relative RMS <= 0.035, element-wise bar); causal, LSE, split key ranges and
per-segment scales at 64 channels too.  The oracle is written for any head
size (its pins include D = 1, 3, 4 and 128).
"""
import numpy as np
import pytest
import torch

import fp8_flash_attention_amd as fa
from oracle import attention as A
from oracle import compare
from oracle import quantize as Qz
from workloads import WORKLOADS, generate, make_workload, sample_rows
from tests.gpu_helpers import check_lse, log, read_codes

pytestmark = pytest.mark.gpu

DIAG_BAR = 0.035


def _run(w, lse=False, causal=False, segment_scales=False):
    q, k, v = generate(w, device="cuda")
    log(f"d64 {w.name} T={w.tokens} H={w.heads} cu={list(w.cu_seqlens)[:8]} lse={lse} causal={causal} "
        f"segment_scales={segment_scales}")
    plan = fa.Plan(w.tokens, w.heads, w.cu_seqlens, w.softmax_scale, device=0, head_dim=64, causal=causal,
                   segment_scales=segment_scales)
    ws = plan.new_workspace()
    ws.fill_(0xFF)
    fa.quantize(plan, q, k, v, ws)
    l = torch.empty((w.heads, w.tokens), dtype=torch.float32, device="cuda") if lse else None
    out = torch.full((w.tokens, w.heads, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    fa.forward(plan, ws, out, l)
    torch.cuda.synchronize()
    return plan, ws, out, l, (q.cpu(), k.cpu(), v.cpu())


def _quantized(q, k, v, cu, sc, segment_scales=False):
    if segment_scales:
        r = Qz.quantize_segments(q, k, v, cu, sc)
        return r, [Qz.dequantize_segments(r[n], r["scales"][i], cu) for i, n in
                   enumerate(("q_codes", "k_codes", "v_codes"))]
    r = Qz.quantize(q, k, v, cu, sc)
    return r, [Qz.dequantize(r[n], r["scales"][i]) for i, n in enumerate(("q_codes", "k_codes", "v_codes"))]


def _check(w, rows, heads=None, causal=False, segment_scales=False, codes=True):
    plan, ws, out, _, (q, k, v) = _run(w, causal=causal, segment_scales=segment_scales)
    hs = list(range(w.heads)) if heads is None else list(heads)
    q, k, v = q[:, hs], k[:, hs], v[:, hs]
    r, (dq, dk, dv) = _quantized(q, k, v, w.cu_seqlens, w.softmax_scale, segment_scales)
    if codes:
        got = read_codes(plan, ws, hs)
        for name in ("q_codes", "k_codes", "v_codes"):
            assert np.array_equal(got[name], r[name]), name
        assert np.array_equal(np.asarray(got["scales"])[..., hs].view(np.uint32), r["scales"].view(np.uint32))
        assert np.array_equal(got["mu"][:, hs].view(np.uint32), r["mu"].view(np.uint32))
        for name, pad in got["pads"].items():
            assert not pad.size or not pad.any(), f"{name} padding bytes not zero"
    o = out.cpu()[:, hs][rows].double().numpy()
    assert np.isfinite(o).all()
    ref = A.attention_rows(q, k, v, w.cu_seqlens, w.softmax_scale, rows, causal=causal).numpy()
    diag = A.attention_rows(dq, dk, dv, w.cu_seqlens, w.softmax_scale, rows, causal=causal).numpy()
    rr, rd = compare.rel_rms(o, ref), compare.rel_rms(o, diag)
    ex_d = compare.allclose_excess(o, diag)
    # rows that see at least 64 keys meet the element-wise bar against the exact inputs
    pos = np.array([rw - max(a for a in w.cu_seqlens[:-1] if a <= rw) for rw in rows])
    seglen = np.array([min(b for b in w.cu_seqlens[1:] if b > rw) - max(a for a in w.cu_seqlens[:-1] if a <= rw)
                       for rw in rows])
    wide = (pos >= 64) if causal else (seglen >= 64)
    ex = compare.allclose_excess(o[wide], ref[wide]) if wide.any() else 0.0
    log(f"  rel_rms={rr:.5f} diagnostic={rd:.5f} excess vs dequantized={ex_d:.5f} vs exact (>= 64 keys)={ex:.5f}")
    assert rr <= compare.REL_RMS_BAR and rd <= DIAG_BAR and ex_d <= 0.0 and ex <= 0.0
    return plan, ws, out


SMALL = [
    make_workload("d64_s256", 256, 2, [0, 256], seed=501, head_dim=64),
    make_workload("d64_ragged", 700, 4, [0, 300, 700], seed=502, k_offset_var=2.0, head_dim=64),
    make_workload("d64_varlen", 1500, 3, [0, 0, 1, 64, 65, 193, 700, 700, 1500], seed=503, head_dim=64),
    make_workload("d64_fused", 500, 4, [0, 130, 500], seed=504, layout="fused", head_dim=64),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_d64_every_element(w):
    _check(w, list(range(w.tokens)))


@pytest.mark.parametrize("w", SMALL[:3], ids=lambda w: w.name)
def test_d64_causal_every_element(w):
    _check(w, list(range(w.tokens)), causal=True, codes=False)


def test_d64_segment_scales():
    w = SMALL[2]
    _check(w, list(range(w.tokens)), segment_scales=True)


def test_d64_full_size_sampled_rows():
    w = WORKLOADS["s30272_h56_d64"]
    rows = sample_rows(w.tokens, 160, seed=w.seed + 7, cu_seqlens=w.cu_seqlens)
    _check(w, rows, heads=[0, 27, 55])


def test_d64_split_keys_lse_and_repeat():
    """A 7-head plan whose last round of work items is split along the keys."""
    w = make_workload("d64_split", 4096, 7, [0, 4096], seed=505, k_offset_var=2.0, head_dim=64)
    plan, ws, out, lse, (q, k, v) = _run(w, lse=True)
    assert plan.info()["partial_slots"] > 0
    l2 = torch.empty_like(lse)
    out2 = fa.forward(plan, ws, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, l2)
    rows = sample_rows(w.tokens, 256, seed=9, cu_seqlens=w.cu_seqlens)
    o = out.cpu()[rows].double().numpy()
    ref = A.attention_rows(q, k, v, w.cu_seqlens, w.softmax_scale, rows).numpy()
    assert compare.rel_rms(o, ref) <= compare.REL_RMS_BAR and compare.allclose_excess(o, ref) <= 0.0
    r, (dq, dk, dv) = _quantized(q, k, v, w.cu_seqlens, w.softmax_scale)
    for s, (a, b) in enumerate(zip(w.cu_seqlens[:-1], w.cu_seqlens[1:])):
        dk[a:b] += r["mu"][s][None].astype(np.float64)
    diag = A.lse_rows(torch.from_numpy(dq), torch.from_numpy(dk), w.cu_seqlens, w.softmax_scale, rows).numpy().T
    check_lse(lse.cpu().double().numpy()[:, rows], diag, False, "head_dim 64 split")


def test_d64_through_attention_wrapper():
    w = SMALL[1]
    q, k, v = generate(w, device="cuda")
    out = fa.attention(q, k, v, cu_seqlens=w.cu_seqlens)
    torch.cuda.synchronize()
    assert out.shape == (w.tokens, w.heads, 64)
    ref = A.attention(q.cpu(), k.cpu(), v.cpu(), w.cu_seqlens, 0.125).numpy()
    assert compare.rel_rms(out.cpu().double().numpy(), ref) <= compare.REL_RMS_BAR


def test_d64_codes_with_more_chunks_than_finalize_threads():
    """More 256-token statistics chunks (70) than the 64 threads of a finalize
    block: every chunk's partial amax must reach the scales."""
    w = make_workload("d64_chunks", 17920, 3, [0, 9000, 17920], seed=506, k_offset_var=2.0, head_dim=64)
    plan, ws, out, _, (q, k, v) = _run(w)
    r, _ = _quantized(q, k, v, w.cu_seqlens, w.softmax_scale)
    got = read_codes(plan, ws)
    assert np.array_equal(got["scales"].view(np.uint32), r["scales"].view(np.uint32))
    for name in ("q_codes", "k_codes", "v_codes"):
        assert np.array_equal(got[name], r[name]), name
