"""GPU parity of plans with a head size other than 64 and 128
(FP8ATTN_PLAN_HEAD_DIM(d), d a multiple of 8 up to 128) against the CPU
oracle, which is written for any head size.  The kernels run at the width 64
or 128 with the missing channels as zeros, so: the codes, scales and K means
of the d real channels must equal the oracle's for d-channel inputs bit for
bit, the padding channels must hold zero codes and zero means, and the output
(d channels only; the rest of a wider output buffer untouched) is graded with
the bars of the 128-channel path: relative RMS <= 0.06 and |o - r| <= 0.1 +
0.1 |r| against the exact inputs (rows that see >= 64 keys), and relative RMS
<= 0.035 and the element-wise bar against the oracle on the dequantized
operands.  Causal plans, the LSE (with the log-linear bound of
tests/gpu_helpers.check_lse) and split key ranges as well.
"""
import numpy as np
import pytest
import torch

import fp8_flash_attention_amd as fa
from oracle import attention as A
from oracle import compare
from workloads import generate, make_workload, sample_rows
from tests.gpu_helpers import check_lse, log, read_codes
from tests.test_gpu_headdim64 import DIAG_BAR, _quantized

pytestmark = pytest.mark.gpu


def _run(w, lse=False, causal=False, wide_out=False):
    D = w.head_dim
    q, k, v = generate(w, device="cuda")
    plan = fa.Plan(w.tokens, w.heads, w.cu_seqlens, w.softmax_scale, device=0, head_dim=D, causal=causal)
    log(f"head_dim {D} {w.name} T={w.tokens} H={w.heads} cu={list(w.cu_seqlens)[:8]} lse={lse} causal={causal} "
        f"pieces={plan.info()['partial_slots']}")
    ws = plan.new_workspace()
    ws.fill_(0xFF)
    fa.quantize(plan, q, k, v, ws)
    l = torch.full((w.heads, w.tokens), float("nan"), dtype=torch.float32, device="cuda") if lse else None
    # the output is a view into a buffer 16 channels wider: nothing past the d
    # channels of a row may be written
    big = torch.full((w.tokens, w.heads, D + 16), 7.0, dtype=torch.bfloat16, device="cuda")
    out = big[:, :, :D]
    fa.forward(plan, ws, out, l)
    torch.cuda.synchronize()
    assert bool((big[:, :, D:] == 7.0).all()), "channels past head_dim were written"
    return plan, ws, out, l, (q.cpu(), k.cpu(), v.cpu())


def _check(w, rows, causal=False, codes=True, lse=False):
    D = w.head_dim
    plan, ws, out, l, (q, k, v) = _run(w, causal=causal, lse=lse)
    r, (dq, dk, dv) = _quantized(q, k, v, w.cu_seqlens, w.softmax_scale)
    if codes:
        got = read_codes(plan, ws)
        for name in ("q_codes", "k_codes", "v_codes"):
            assert np.array_equal(got[name][..., :D], r[name]), name
            assert not got[name][..., D:].any(), f"{name}: padding channels not zero"
        assert np.array_equal(np.asarray(got["scales"]).view(np.uint32), r["scales"].view(np.uint32))
        assert np.array_equal(got["mu"][..., :D].view(np.uint32), r["mu"].view(np.uint32))
        assert not got["mu"][..., D:].any()
    o = out.cpu()[rows].double().numpy()
    assert np.isfinite(o).all()
    ref = A.attention_rows(q, k, v, w.cu_seqlens, w.softmax_scale, rows, causal=causal).numpy()
    diag = A.attention_rows(dq, dk, dv, w.cu_seqlens, w.softmax_scale, rows, causal=causal).numpy()
    rr, rd = compare.rel_rms(o, ref), compare.rel_rms(o, diag)
    ex_d = compare.allclose_excess(o, diag)
    pos = np.array([rw - max(a for a in w.cu_seqlens[:-1] if a <= rw) for rw in rows])
    seglen = np.array([min(b for b in w.cu_seqlens[1:] if b > rw) - max(a for a in w.cu_seqlens[:-1] if a <= rw)
                       for rw in rows])
    wide = (pos >= 64) if causal else (seglen >= 64)
    ex = compare.allclose_excess(o[wide], ref[wide]) if wide.any() else 0.0
    log(f"  rel_rms={rr:.5f} diagnostic={rd:.5f} excess vs dequantized={ex_d:.5f} vs exact (>= 64 keys)={ex:.5f}")
    assert rr <= compare.REL_RMS_BAR and rd <= DIAG_BAR and ex_d <= 0.0 and ex <= 0.0
    if lse:
        dkc = dk.copy()
        for s, (a, b) in enumerate(zip(w.cu_seqlens[:-1], w.cu_seqlens[1:])):
            dkc[a:b] += r["mu"][s][None].astype(np.float64)
        ld = A.lse_rows(torch.from_numpy(dq), torch.from_numpy(dkc), w.cu_seqlens, w.softmax_scale, rows,
                        causal=causal).numpy().T
        check_lse(l.cpu().double().numpy()[:, rows], ld, False, f"head_dim {D}")
    return plan


@pytest.mark.parametrize("d", [8, 32, 72, 96, 120])
def test_head_dim_every_element(d):
    w = make_workload(f"d{d}_varlen", 1200, 3, [0, 0, 1, 64, 65, 193, 700, 700, 1200], seed=600 + d,
                      k_offset_var=2.0, head_dim=d)
    _check(w, list(range(w.tokens)), lse=True)


@pytest.mark.parametrize("d", [40, 96])
def test_head_dim_causal_every_element(d):
    w = make_workload(f"d{d}_causal", 700, 3, [0, 300, 700], seed=650 + d, head_dim=d)
    _check(w, list(range(w.tokens)), causal=True, codes=False, lse=True)


def test_head_dim_split_keys_every_element():
    w = make_workload("d96_split", 2000, 8, [0, 1000, 2000], seed=660, k_offset_var=2.0, head_dim=96)
    plan = _check(w, list(range(w.tokens)), lse=True)
    assert plan.info()["partial_slots"] > 0


def test_head_dim_full_size_sampled():
    w = make_workload("d96_s4096_h56", 4096, 56, [0, 4096], seed=670, k_offset_var=2.0, head_dim=96)
    rows = sample_rows(w.tokens, 256, seed=671, cu_seqlens=w.cu_seqlens)
    _check(w, rows, codes=False)


def test_head_dim_through_the_binding():
    """fa.attention takes the head size from the inputs."""
    w = make_workload("d80_binding", 500, 2, [0, 200, 500], seed=680, head_dim=80)
    q, k, v = generate(w, device="cuda")
    log("head_dim 80 through fa.attention")
    o = fa.attention(q, k, v, cu_seqlens=w.cu_seqlens)
    torch.cuda.synchronize()
    assert o.shape == (500, 2, 80)
    ref = A.attention(q.cpu(), k.cpu(), v.cpu(), w.cu_seqlens, w.softmax_scale).numpy()
    assert compare.rel_rms(o.cpu().double().numpy(), ref) <= compare.REL_RMS_BAR
