"""GPU parity of E4M3 plans made with FP8ATTN_PLAN_EXACT_PROBS (probabilities
rounded from the FP32 exp2, the pages' recipe) against the float64 oracle,
with the bars of tests/test_gpu_attention.py: every element of small and edge
cases, sampled rows at full size with the kernel-only bar on three heads,
split items, the LSE (the log of the applied weights, as for default plans)
and causal plans."""
import numpy as np
import pytest
import torch

import fp8_flash_attention_amd as fa
from oracle import attention as A
from oracle import compare
from oracle import quantize as Qz
from workloads import WORKLOADS, generate, make_workload, sample_rows
from tests.gpu_helpers import check_lse, log
from tests.test_gpu_attention import DIAG_BAR, _check_rows, _dequantized, _gpu_attention

pytestmark = pytest.mark.gpu


def test_s256_h2_every_element():
    w = WORKLOADS["s256_h2"]
    got, (q, k, v) = _check_rows(w, list(range(w.tokens)), pure_atol=True, exact=True)
    dq, dk, dv = _dequantized(q, k, v, w.cu_seqlens, w.softmax_scale)
    assert compare.rel_rms(got, A.attention(dq, dk, dv, w.cu_seqlens, w.softmax_scale).numpy()) <= DIAG_BAR


@pytest.mark.parametrize("name,nrows", [("s4096_h56", 256), ("s30272_h56_koffset", 192), ("varlen_30272_h56", 192)])
def test_full_size_sampled_rows(name, nrows):
    w = WORKLOADS[name]
    rows = sample_rows(w.tokens, nrows, seed=w.seed + 27, cu_seqlens=w.cu_seqlens)
    got, (q, k, v) = _check_rows(w, rows, pure_atol=len(w.segments) == 1, exact=True)
    hs = [0, 31, 55]
    dq, dk, dv = _dequantized(q[:, hs], k[:, hs], v[:, hs], w.cu_seqlens, w.softmax_scale)
    diag = A.attention_rows(dq, dk, dv, w.cu_seqlens, w.softmax_scale, rows).numpy()
    rr = compare.rel_rms(got[:, hs], diag)
    log(f"  diagnostic rel_rms={rr:.5f}")
    assert rr <= DIAG_BAR


@pytest.mark.parametrize("cu", [[0, 1, 1, 64, 65, 200, 200, 457], [0, 3000]])
def test_edge_and_split_every_element(cu):
    w = make_workload("exact_edge", cu[-1], 2, cu, seed=131)
    _check_rows(w, list(range(w.tokens)), exact=True)


def test_lse_and_log_linear_default_agree_closely():
    # the two probability encodings differ by the encoding alone: outputs within
    # the kernel-only error of each other; each plan's LSE is the log of the
    # weights it applied (its normalizer), within its code's error range of the
    # exact log-sum-exp of the dequantized operands
    w = make_workload("exact_lse", 1000, 3, [0, 400, 1000], seed=132, k_offset_var=2.0)
    q, k, v = generate(w, device="cuda")
    _, _, o_e, l_e = _gpu_attention(w, q, k, v, lse=True, exact=True)
    _, _, o_d, l_d = _gpu_attention(w, q, k, v, lse=True, exact=False)
    assert compare.rel_rms(o_d.cpu().double().numpy(), o_e.cpu().double().numpy()) <= 0.06
    r = Qz.quantize(q.cpu(), k.cpu(), v.cpu(), w.cu_seqlens, w.softmax_scale)
    dq = Qz.dequantize(r["q_codes"], r["scales"][0])
    dk = Qz.dequantize(r["k_codes"], r["scales"][1])
    for s, (a, b) in enumerate(zip(w.cu_seqlens[:-1], w.cu_seqlens[1:])):
        dk[a:b] += r["mu"][s][None].astype(np.float64)
    ld = A.lse_rows(torch.from_numpy(dq), torch.from_numpy(dk), w.cu_seqlens, w.softmax_scale).numpy().T
    check_lse(l_e.cpu().double().numpy(), ld, True, "exact")
    check_lse(l_d.cpu().double().numpy(), ld, False, "default")


def test_causal_exact_probs():
    w = make_workload("exact_causal", 700, 2, [0, 300, 700], seed=133)
    q, k, v = generate(w, device="cuda")
    plan = fa.Plan(w.tokens, w.heads, w.cu_seqlens, w.softmax_scale, device=0, causal=True, exact_probs=True)
    ws = plan.new_workspace()
    fa.quantize(plan, q, k, v, ws)
    out = fa.forward(plan, ws)
    torch.cuda.synchronize()
    ref = A.attention(q.cpu(), k.cpu(), v.cpu(), w.cu_seqlens, w.softmax_scale, causal=True).numpy()
    assert compare.rel_rms(out.cpu().double().numpy(), ref) <= compare.REL_RMS_BAR


def test_exact_probs_rejected_for_fp4_plans():
    with pytest.raises(fa.Fp8AttnError):
        fa.Plan(256, 2, [0, 256], device=0, fmt="mxfp4", exact_probs=True)
