"""Seeded random plan configurations through the library, each against the
oracle (test infrastructure; the bars are those of the targeted tests).

E4M3 plans draw the segment table (empty, one-token, tile-edge and longer
segments), the head count, the head size (any multiple of 8 up to 128), and
whether the plan is causal, has per-segment scales, exact probabilities, a
K offset and Q block-mean centring.  Each checks: the E4M3 codes, scales and K means of the real
channels bit for bit (padding channels zero); every output element against
the oracle on the dequantized operands (with Q centring: the centred codes
plus the exact block mean) (|o - r| <= 0.1 + 0.1 |r|, relative
RMS <= 0.035 over rows that see >= 64 keys); rows that see >= 64 keys
against the exact inputs with the same element-wise bar; the LSE with
tests/gpu_helpers.check_lse.

FP4 plans draw the segment table, head count, causal and Q centring, and
check every output element and the LSE against the FP4 reference's own
computation (the bars of tests/test_gpu_mxfp4.py).
"""
import numpy as np
import pytest
import torch

import fp8_flash_attention_amd as fa
from oracle import attention as A
from oracle import compare
from oracle import mxfp4 as M
from oracle import quantize as Qz
from workloads import generate, make_workload
from tests.cases import FEW_KEYS, visible_keys
from tests.gpu_helpers import check_lse, log, read_codes
from tests.test_gpu_mxfp4 import _check_output, check_lse_values

pytestmark = pytest.mark.gpu

LENGTHS = [0, 1, 7, 63, 64, 65, 127, 128, 200, 257, 400, 700]


def _table(rng):
    lens = [int(x) for x in rng.choice(LENGTHS, size=int(rng.integers(1, 6)))]
    if sum(lens) == 0:
        lens.append(100)
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    return cu


def _e4m3_config(i):
    rng = np.random.default_rng(9100 + i)
    cu = _table(rng)
    c = dict(cu=cu, H=int(rng.integers(1, 5)), D=8 * int(rng.integers(1, 17)), causal=bool(rng.random() < 0.4),
             seg=bool(rng.random() < 0.3), exact=bool(rng.random() < 0.3),
             koff=2.0 if rng.random() < 0.5 else None, seed=9100 + i)
    c["qc"] = bool(rng.random() < 0.5)     # drawn last: the other draws are unchanged
    return c


@pytest.mark.parametrize("i", range(16))
def test_random_e4m3_config(i):
    c = _e4m3_config(i)
    cu, H, D = c["cu"], c["H"], c["D"]
    w = make_workload(f"rand{i}", cu[-1], H, cu, seed=c["seed"], k_offset_var=c["koff"], head_dim=D)
    log(f"random e4m3 #{i}: cu={cu} H={H} D={D} causal={c['causal']} segment_scales={c['seg']} "
        f"exact={c['exact']} k_offset={c['koff']} q_centre={c['qc']}")
    q, k, v = generate(w, device="cuda")
    plan = fa.Plan(w.tokens, H, cu, w.softmax_scale, device=0, head_dim=D, causal=c["causal"],
                   segment_scales=c["seg"], exact_probs=c["exact"], q_centre=c["qc"])
    ws = plan.new_workspace()
    ws.fill_(0xFF)
    fa.quantize(plan, q, k, v, ws)
    lse = torch.full((H, w.tokens), float("nan"), dtype=torch.float32, device="cuda")
    out = fa.forward(plan, ws, lse=lse)
    torch.cuda.synchronize()
    q, k, v = q.cpu(), k.cpu(), v.cpu()
    if c["seg"]:
        r = Qz.quantize_segments(q, k, v, cu, w.softmax_scale, q_centre=c["qc"])
        deq = [Qz.dequantize_segments(r[n], r["scales"][j], cu) for j, n in enumerate(("q_codes", "k_codes", "v_codes"))]
    else:
        r = Qz.quantize(q, k, v, cu, w.softmax_scale, q_centre=c["qc"])
        deq = [Qz.dequantize(r[n], r["scales"][j]) for j, n in enumerate(("q_codes", "k_codes", "v_codes"))]
    if c["qc"]:
        deq[0] = Qz.qcentre_operand(r["q_codes"], r["scales"][0], r["qm"], cu)
    got = read_codes(plan, ws)
    for name in ("q_codes", "k_codes", "v_codes"):
        assert np.array_equal(got[name][..., :D], r[name]), name
        assert not got[name][..., D:].any(), name
    assert np.array_equal(np.asarray(got["scales"]).reshape(r["scales"].shape).view(np.uint32),
                          r["scales"].view(np.uint32))
    assert np.array_equal(got["mu"][..., :D].view(np.uint32), r["mu"].view(np.uint32))
    o = out.cpu().double().numpy()
    assert np.isfinite(o).all()
    dq, dk, dv = deq
    diag = A.attention(dq, dk, dv, cu, w.softmax_scale, causal=c["causal"]).numpy()
    ref = A.attention(q, k, v, cu, w.softmax_scale, causal=c["causal"]).numpy()
    wide = visible_keys(cu, c["causal"]) >= FEW_KEYS
    ex_d = compare.allclose_excess(o, diag)
    rd = compare.rel_rms(o[wide], diag[wide]) if wide.any() else 0.0
    ex = compare.allclose_excess(o[wide], ref[wide]) if wide.any() else -1.0
    log(f"  vs dequantized: excess {ex_d:.4f}, rel_rms (>= 64 keys) {rd:.4f}; vs exact (>= 64 keys) excess {ex:.4f}")
    assert ex_d <= 0.0 and rd <= 0.035 and ex <= 0.0
    dkc = dk.copy()
    for s, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        dkc[a:b] += r["mu"][s][None].astype(np.float64)
    ld = A.lse_rows(torch.from_numpy(dq), torch.from_numpy(dkc), cu, w.softmax_scale, causal=c["causal"]).numpy().T
    check_lse(lse.cpu().double().numpy(), ld, c["exact"], "random")


@pytest.mark.parametrize("i", range(8))
def test_random_fp4_config(i):
    rng = np.random.default_rng(9300 + i)
    cu = _table(rng)
    H = int(rng.integers(1, 4))
    causal, qc = bool(rng.random() < 0.5), bool(rng.random() < 0.5)
    w = make_workload(f"rand_mx{i}", cu[-1], H, cu, seed=9300 + i, k_offset_var=2.0 if rng.random() < 0.5 else None)
    log(f"random fp4 #{i}: cu={cu} H={H} causal={causal} q_centre={qc}")
    q, k, v = generate(w, device="cuda")
    plan = fa.Plan(w.tokens, H, cu, w.softmax_scale, device=0, fmt="mxfp4", q_centre=qc, causal=causal)
    ws = plan.new_workspace()
    ws.fill_(0xFF)
    fa.quantize(plan, q, k, v, ws)
    lse = torch.full((H, w.tokens), float("nan"), dtype=torch.float32, device="cuda")
    out = fa.forward(plan, ws, lse=lse)
    torch.cuda.synchronize()
    q, k, v = q.cpu(), k.cpu(), v.cpu()
    z = M.quantize_mxfp4(q, k, v, cu, w.softmax_scale, q_centre=qc)
    ops = M.dequantized_operands(z, cu)
    ref = M.attention_from_operands(ops["Q"], ops["QM"], ops["K"], ops["V"], cu, causal=causal)
    o = out.float().cpu().numpy()
    assert np.isfinite(o).all()
    _check_output(o, ref, w.name)
    lref = M.lse_mxfp4_rows(z, cu, list(range(w.tokens)), list(range(H)), causal=causal)
    check_lse_values(lse.cpu().double().numpy().T, lref, w.name)
