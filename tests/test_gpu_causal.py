"""GPU parity of causal plans (FP8ATTN_PLAN_CAUSAL) against the float64 oracle's
causal reading (query i of a segment attends keys j <= i of it).

Bars as for the non-causal path: relative RMS <= 0.06 against the exact
inputs and <= 0.035 against the oracle on the dequantized E4M3 operands; the
element-wise |o - r| <= 0.1 + 0.1 |r| against the exact inputs for rows that
see at least 64 keys, and against the dequantized-operand oracle for every
row (rows near a segment start average a few V rows; see ``_check``).  Small cases compare
every element (segments of every length class: one token, shorter than a
tile, a partial last tile, several 256-query items, empty segments); the
full sizes compare sampled rows.  A segment's first row sees one key, so its
output is that key's dequantized V row up to the BF16 rounding.
"""
import numpy as np
import pytest
import torch

import fp8_flash_attention_amd as fa
from oracle import attention as A
from oracle import compare
from oracle import quantize as Qz
from workloads import WORKLOADS, generate, make_workload, sample_rows
from tests.cases import CAUSAL_CASES, FEW_KEYS, visible_keys
from tests.gpu_helpers import check_lse, bf16_ulp, log

pytestmark = pytest.mark.gpu

DIAG_BAR = 0.035


def _run(w, lse=False):
    q, k, v = generate(w, device="cuda")
    log(f"causal {w.name} T={w.tokens} H={w.heads} cu={list(w.cu_seqlens)[:8]} lse={lse}")
    plan = fa.Plan(w.tokens, w.heads, w.cu_seqlens, w.softmax_scale, device=0, causal=True)
    assert plan.info()["causal"] == 1 and plan.info()["partial_slots"] == 0
    ws = plan.new_workspace()
    fa.quantize(plan, q, k, v, ws)
    l = torch.empty((w.heads, w.tokens), dtype=torch.float32, device="cuda") if lse else None
    out = torch.full((w.tokens, w.heads, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    fa.forward(plan, ws, out, l)
    torch.cuda.synchronize()
    return plan, ws, out, l, (q.cpu(), k.cpu(), v.cpu())


def _dequantized(q, k, v, cu, softmax_scale):
    r = Qz.quantize(q, k, v, cu, softmax_scale)
    sc = r["scales"]
    return (Qz.dequantize(r["q_codes"], sc[0]), Qz.dequantize(r["k_codes"], sc[1]),
            Qz.dequantize(r["v_codes"], sc[2]), r)


def _check(w, rows, heads=None):
    plan, ws, out, _, (q, k, v) = _run(w)
    hs = list(range(w.heads)) if heads is None else list(heads)
    q, k, v = q[:, hs], k[:, hs], v[:, hs]
    got = out.cpu()[:, hs][rows].double().numpy()
    assert np.isfinite(got).all()
    ref = A.attention_rows(q, k, v, w.cu_seqlens, w.softmax_scale, rows, causal=True).numpy()
    rr = compare.rel_rms(got, ref)
    dq, dk, dv, _ = _dequantized(q, k, v, w.cu_seqlens, w.softmax_scale)
    diag = A.attention_rows(dq, dk, dv, w.cu_seqlens, w.softmax_scale, rows, causal=True).numpy()
    rd = compare.rel_rms(got, diag)
    # Rows near a segment start average a handful of V rows with E4M3-rounded
    # weights: there the FP8 recipe itself (oracle.attention_fp8_recipe, no
    # kernel involved) breaks the element-wise bar against the exact inputs
    # (tests/test_oracle_fp8_recipe.py shows it on these very cases), so such
    # rows are held to the bar against the oracle on the dequantized operands
    # (the kernel's own error); rows that see at least FEW_KEYS keys meet it
    # against the exact inputs.
    wide = visible_keys(w.cu_seqlens, True)[rows] >= FEW_KEYS
    ex_d = compare.allclose_excess(got, diag)
    ex = compare.allclose_excess(got[wide], ref[wide]) if wide.any() else 0.0
    log(f"  rel_rms={rr:.5f} diagnostic rel_rms={rd:.5f} allclose_excess: vs dequantized {ex_d:.5f}, "
        f"rows with >= 64 keys vs exact {ex:.5f}")
    assert rr <= compare.REL_RMS_BAR and rd <= DIAG_BAR and ex_d <= 0.0 and ex <= 0.0
    # the first row of every segment is its first key's dequantized V row
    for a, b in zip(w.cu_seqlens[:-1], w.cu_seqlens[1:]):
        if b > a and a in rows:
            i = rows.index(a)
            assert np.all(np.abs(got[i] - dv[a]) <= bf16_ulp(dv[a]) / 2 + 1e-6)
    return plan, ws, out


CASES = CAUSAL_CASES


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_causal_every_element(w):
    _check(w, list(range(w.tokens)))


@pytest.mark.parametrize("name,nrows", [("s4096_h56", 256), ("varlen_30272_h56", 192), ("s30272_h56_koffset", 160)])
def test_causal_full_size_sampled_rows(name, nrows):
    w = WORKLOADS[name]
    rows = sample_rows(w.tokens, nrows, seed=w.seed + 17, cu_seqlens=w.cu_seqlens)
    _check(w, rows, heads=[0, w.heads // 2, w.heads - 1])


def test_causal_lse_and_repeat():
    w = make_workload("c_lse", 900, 3, [0, 100, 100, 900], seed=405, k_offset_var=2.0)
    plan, ws, out, lse, (q, k, v) = _run(w, lse=True)
    l2 = torch.empty_like(lse)
    out2 = fa.forward(plan, ws, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, l2)
    _, dk, _, r = _dequantized(q, k, v, w.cu_seqlens, w.softmax_scale)
    dq = Qz.dequantize(r["q_codes"], r["scales"][0])
    for s, (a, b) in enumerate(zip(w.cu_seqlens[:-1], w.cu_seqlens[1:])):
        dk[a:b] += r["mu"][s][None].astype(np.float64)
    diag = A.lse_rows(torch.from_numpy(dq), torch.from_numpy(dk), w.cu_seqlens, w.softmax_scale,
                      causal=True).numpy().T
    check_lse(lse.cpu().double().numpy(), diag, False, "causal")


def test_batched_input_through_the_binding():
    """[B, T, H, D] views run as B segments; causal and not."""
    B, T, H = 3, 200, 2
    w = make_workload("batch", B * T, H, [0, T, 2 * T, 3 * T], seed=406)
    q, k, v = generate(w, device="cuda")
    for causal in (False, True):
        log(f"batched B={B} T={T} causal={causal}")
        o4 = fa.attention(q.view(B, T, H, 128), k.view(B, T, H, 128), v.view(B, T, H, 128), causal=causal)
        o3 = fa.attention(q, k, v, cu_seqlens=w.cu_seqlens, causal=causal)
        torch.cuda.synchronize()
        assert o4.shape == (B, T, H, 128)
        assert torch.equal(o4.view(B * T, H, 128), o3)
        ref = A.attention(q.cpu(), k.cpu(), v.cpu(), w.cu_seqlens, w.softmax_scale, causal=causal).numpy()
        assert compare.rel_rms(o3.cpu().double().numpy(), ref) <= compare.REL_RMS_BAR

