"""GPU parity of the block-scaled FP4 variant (plans made with fmt="mxfp4")
against the CPU reference ``oracle.mxfp4``.

* Codes and block scales of Q, K, V and of the Q block-mean operand, and the K
  means: bit for bit, every element of the small cases, sampled heads at the
  full sizes (quantization is per head).
* Output: against the reference's own FP4 computation from its quantized
  operands, element by element (bar below), and against the float64 softmax
  attention within the pages' FP4 tolerance (atol 1.0, rtol 0.1) with the
  relative RMS error reported by the reference's pin.
* Inputs for which every quantization step is lossless give the plain softmax
  attention up to BF16 rounding.
* The LSE output, key splits (with the combine pass) and causal plans against
  the reference's readings 8 and 9.

Element-wise bar against the reference's FP4 computation: the scores are
exact in both (E2M1 products with power-of-two scales, float32 sums that do
not round for these magnitudes); the probabilities come from the kernel's
exp2, which is within an ulp or two of 2^x, so an E2M1 probability code can
flip only where 2^(x-E) lies within that of a rounding midpoint (about one
element in 10^6); the rest is float32 accumulation and one BF16 rounding.
Bar: |gpu - ref| <= 2 BF16 ulps of |ref| + 2^-10 * max|ref| of the row, with
at most 1e-4 of the elements (code flips) allowed up to 0.05 * max|ref| of
the row.
"""
import numpy as np
import pytest
import torch

import fp8_flash_attention_amd as fa
from fp8_flash_attention_amd import _lib
from oracle import attention as exact
from oracle import mxfp4 as M
from workloads import WORKLOADS, generate, make_workload, sample_rows
from tests.cases import FEW_KEYS, visible_keys
from tests.gpu_helpers import log, bf16_ulp

pytestmark = pytest.mark.gpu

POS = np.array([0, 2, 1, 3])          # byte position of channel block j in a row's scale bytes


def _unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """uint8 [..., n] -> codes [..., 2n] (low nibble first)."""
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.uint8)
    out[..., 0::2] = b & 15
    out[..., 1::2] = b >> 4
    return out


def _rows_of_tokens(cu):
    row = np.zeros(cu[-1], np.int64)
    r0 = 0
    row0 = []
    for a, b in zip(cu[:-1], cu[1:]):
        row[a:b] = r0 + np.arange(b - a)
        row0.append(r0)
        r0 += (b - a + 127) // 128 * 128
    return row, row0


def read_mx(plan, ws, heads):
    """GPU workspace in the reference's layout (see ``oracle.mxfp4.quantize_mxfp4``)."""
    cu = list(plan.cu_seqlens)
    hs = list(heads)
    row, row0 = _rows_of_tokens(cu)
    get = lambda which: plan.region(ws, which)[hs].cpu().numpy()
    qc, kc, vc = get(_lib.REGION_Q), get(_lib.REGION_K), get(_lib.REGION_V)
    qs, ks, vs = get(_lib.REGION_Q_BSCALES), get(_lib.REGION_K_BSCALES), get(_lib.REGION_V_BSCALES)
    mc, ms = get(_lib.REGION_QM_CODES), get(_lib.REGION_QM_SCALES)
    out = {}
    out["q_codes"] = _unpack_nibbles(qc[:, row]).transpose(1, 0, 2)
    out["k_codes"] = _unpack_nibbles(kc[:, row]).transpose(1, 0, 2)
    out["q_e"] = qs[:, row][:, :, POS].astype(np.int64).transpose(1, 0, 2) - 127
    out["k_e"] = ks[:, row][:, :, POS].astype(np.int64).transpose(1, 0, 2) - 127
    # V: tile t, channel d, byte i -> keys 64t + 2i, 64t + 2i + 1
    vt = _unpack_nibbles(vc.reshape(len(hs), -1, 128, 32))          # [H, tiles, 128, 64]
    vrow = vt.transpose(0, 1, 3, 2).reshape(len(hs), -1, 128)       # [H, rows, 128]
    out["v_codes"] = vrow[:, row].transpose(1, 0, 2)
    ve = []
    for s, a, b in M.v_blocks(cu):
        r = row0[s] + (a - cu[s])
        t, kb = r // 64, (r % 64) // 32
        d = np.arange(128)
        ve.append(vs[:, t, (32 * kb + d % 32) * 4 + d // 32].astype(np.int64) - 127)
    out["v_e"] = np.array(ve).reshape(-1, len(hs), 128)
    qb = []
    qbe = []
    for s, a, b in M.q_blocks(cu):
        blk = (row0[s] + (a - cu[s])) // 128
        qb.append(_unpack_nibbles(mc[:, blk]))
        qbe.append(ms[:, blk][:, POS].astype(np.int64) - 127)
    out["qm_codes"] = np.array(qb).reshape(-1, len(hs), 128)
    out["qm_e"] = np.array(qbe).reshape(-1, len(hs), 4)
    out["mu"] = plan.region(ws, _lib.REGION_MU).cpu().numpy()[:, hs]
    return out


def _run(w, q_centre, heads=None, poison=True, causal=False, lse=False):
    q, k, v = generate(w, device="cuda")
    plan = fa.Plan(w.tokens, w.heads, w.cu_seqlens, w.softmax_scale, device=0, fmt="mxfp4", q_centre=q_centre,
                   causal=causal)
    ws = plan.new_workspace()
    if poison:
        ws.fill_(0xFF)
    out = torch.full((w.tokens, w.heads, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    l = torch.full((w.heads, w.tokens), float("nan"), dtype=torch.float32, device="cuda") if lse else None
    log(f"mxfp4 {w.name} T={w.tokens} H={w.heads} cu={w.cu_seqlens[:8]} q_centre={q_centre} causal={causal} "
        f"lse={lse} layout={w.layout} pieces={plan.info()['partial_slots']}")
    fa.quantize(plan, q, k, v, ws)
    fa.forward(plan, ws, out, l)
    torch.cuda.synchronize()
    hs = list(range(w.heads)) if heads is None else list(heads)
    if lse:
        return plan, ws, out, l, (q.cpu()[:, hs], k.cpu()[:, hs], v.cpu()[:, hs]), hs
    return plan, ws, out, (q.cpu()[:, hs], k.cpu()[:, hs], v.cpu()[:, hs]), hs


def _check_codes(got, exp):
    for name in ("q_codes", "k_codes", "v_codes", "q_e", "k_e", "v_e", "qm_codes", "qm_e"):
        a, b = np.asarray(got[name]), np.asarray(exp[name])
        assert a.shape == b.shape, (name, a.shape, b.shape)
        bad = np.argwhere(a != b)
        assert bad.size == 0, f"{name}: {len(bad)} mismatches, first at {bad[0]}: gpu={a[tuple(bad[0])]} " \
                              f"cpu={b[tuple(bad[0])]}"
    assert np.array_equal(got["mu"].view(np.uint32), exp["mu"].view(np.uint32))


def _check_output(o, ref, what):
    """o, ref: [R, H, 128] (BF16 output as float, float64 reference)."""
    rmax = np.abs(ref).max(axis=2, keepdims=True)
    err = np.abs(o - ref)
    tight = 2 * bf16_ulp(ref) + 2.0 ** -10 * rmax
    loose = 0.05 * rmax
    over = err > tight
    assert not np.any(err > loose), f"{what}: max error {err.max():.4g} beyond the code-flip bound"
    assert over.mean() <= 1e-4, f"{what}: {over.sum()} of {over.size} elements above the tight bar " \
                                f"(max excess {(err - tight).max():.3g})"


CASES = [
    make_workload("mx_s256", 256, 2, [0, 256], seed=301),
    make_workload("mx_ragged", 700, 4, [0, 300, 700], seed=302, k_offset_var=2.0),
    make_workload("mx_varlen", 1200, 3, [0, 0, 1, 64, 65, 193, 700, 700, 1200], seed=303),
    make_workload("mx_fused", 500, 4, [0, 130, 500], seed=304, layout="fused"),
]


@pytest.mark.parametrize("q_centre", [True, False])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_mxfp4_codes_and_output_small(w, q_centre):
    plan, ws, out, (q, k, v), hs = _run(w, q_centre)
    z = M.quantize_mxfp4(q, k, v, w.cu_seqlens, w.softmax_scale, q_centre=q_centre)
    _check_codes(read_mx(plan, ws, hs), z)
    ops = M.dequantized_operands(z, w.cu_seqlens)
    ref = M.attention_from_operands(ops["Q"], ops["QM"], ops["K"], ops["V"], w.cu_seqlens)
    o = out.float().cpu().numpy()
    assert np.isfinite(o).all()
    _check_output(o, ref, w.name)
    # and the method's own error against the float64 softmax: the pages' FP4 bar
    ex = exact.attention(q, k, v, w.cu_seqlens, w.softmax_scale).numpy()
    assert np.all(np.abs(o - ex) <= 1.0 + 0.1 * np.abs(ex))
    rel = np.linalg.norm(o - ex) / np.linalg.norm(ex)
    log(f"  rel RMS vs float64 softmax: {rel:.4f}")
    assert rel < 0.35


def test_mxfp4_lossless_inputs_give_the_softmax():
    """The reference pin's lossless construction run through the library."""
    from tests.test_oracle_mxfp4 import SIGMA_C8, _lossless_inputs
    cu = [0, 256, 384]
    q, k, v = _lossless_inputs(cu, 2, seed=9)
    for q_centre in (True, False):
        plan = fa.Plan(384, 2, cu, SIGMA_C8, device=0, fmt="mxfp4", q_centre=q_centre)
        ws = plan.new_workspace()
        log(f"mxfp4 lossless q_centre={q_centre}")
        fa.quantize(plan, q.cuda(), k.cuda(), v.cuda(), ws)
        out = fa.forward(plan, ws)
        torch.cuda.synchronize()
        want = exact.attention(q, k, v, cu, SIGMA_C8).numpy()
        o = out.float().cpu().numpy()
        assert np.all(np.abs(o - want) <= bf16_ulp(want) / 2 + 1e-6)


def test_mxfp4_repeat_is_bit_identical_and_strided_output():
    w = CASES[1]
    plan, ws, out, _, _ = _run(w, True)
    big = torch.zeros((w.tokens, w.heads, 256), dtype=torch.bfloat16, device="cuda")
    view = big[:, :, 64:192]
    fa.forward(plan, ws, view)
    fa.forward(plan, ws, out)
    torch.cuda.synchronize()
    assert torch.equal(view.cpu(), out.cpu())
    assert not big[:, :, :64].any() and not big[:, :, 192:].any()


def test_mxfp4_empty_input():
    p0 = fa.Plan(0, 2, [0, 0], device=0, fmt="mxfp4")
    ws0 = p0.new_workspace()
    z = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    log("mxfp4 empty input with an LSE output")
    fa.quantize(p0, z, z, z, ws0)
    fa.forward(p0, ws0, z, torch.empty((2, 0), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()


# LSE bar: both sides take the same scores (exact, see above) and the log of
# the same quantized weights (the row's normalizer); the kernel's FP32 sums are
# good to a few parts in 1e6, and (Qhat + QMhat) . mu is a 128-term FP32 dot
# product of exact values, so 1e-3 in natural-log units leaves two orders of
# magnitude.  As for the output, the hardware exp2's last bits can move a
# weight to the neighbouring E2M1 value where 2^(x - E) sits on a rounding
# midpoint: such a row moves by at most ln 1.5 (4 <-> 6 in a block whose
# largest weight, in (3, 6], is the only one), and at most 0.1% of the entries
# (two at least) may do so.
LSE_BAR = 1e-3
LSE_FLIP_BAR = float(np.log(1.5)) + 1e-3


def check_lse_values(got: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    """The bar above, on LSE values and their references of the same shape."""
    err = np.abs(np.asarray(got, np.float64) - ref)
    n_off = int((err > LSE_BAR).sum())
    log(f"  {what} lse max err {err.max():.2e}, {n_off} of {err.size} entries above {LSE_BAR}")
    assert np.isfinite(got).all()
    assert err.max() <= LSE_FLIP_BAR
    assert n_off <= max(2, err.size // 1000)


def _check_lse(lse, z, cu, hs, causal=False):
    got = lse.cpu().double().numpy()[hs].T                                  # [T, H]
    ref = M.lse_mxfp4_rows(z, cu, list(range(cu[-1])), list(range(len(hs))), causal=causal)
    check_lse_values(got, ref)


@pytest.mark.parametrize("q_centre", [True, False])
@pytest.mark.parametrize("w", CASES[:3], ids=lambda w: w.name)
def test_mxfp4_lse(w, q_centre):
    """LSE of the uncentred scores (reading 9 of the FP4 reference) for every
    row and head; the output with the LSE variant is the same as without."""
    plan, ws, out, lse, (q, k, v), hs = _run(w, q_centre, lse=True)
    z = M.quantize_mxfp4(q, k, v, w.cu_seqlens, w.softmax_scale, q_centre=q_centre)
    _check_lse(lse, z, list(w.cu_seqlens), hs)
    out2 = fa.forward(plan, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


SPLIT_CASES = [
    make_workload("mx_split", 2048, 4, [0, 2048], seed=311, k_offset_var=2.0),        # four pieces an item
    make_workload("mx_split_ragged", 2000, 4, [0, 2000], seed=312),                  # last piece ends ragged
    make_workload("mx_split_varlen", 2000, 8, [0, 1000, 2000], seed=313),            # two pieces an item
]


@pytest.mark.parametrize("q_centre", [True, False])
@pytest.mark.parametrize("w", SPLIT_CASES, ids=lambda w: w.name)
def test_mxfp4_split_keys_every_element(w, q_centre):
    """Key splits of the last round: every element against the reference's FP4
    computation, the LSE through the combine pass, and bit-identical repeats."""
    plan, ws, out, lse, (q, k, v), hs = _run(w, q_centre, lse=True)
    items = [it for it in plan.work_items() if it[0] >= 0]
    assert items and all(it[3] != 0 for it in items)
    z = M.quantize_mxfp4(q, k, v, w.cu_seqlens, w.softmax_scale, q_centre=q_centre)
    ops = M.dequantized_operands(z, w.cu_seqlens)
    ref = M.attention_from_operands(ops["Q"], ops["QM"], ops["K"], ops["V"], w.cu_seqlens)
    o = out.float().cpu().numpy()
    assert np.isfinite(o).all()
    _check_output(o, ref, w.name)
    _check_lse(lse, z, list(w.cu_seqlens), hs)
    l2 = torch.empty_like(lse)
    out2 = fa.forward(plan, ws, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, l2)


CAUSAL_CASES = [
    make_workload("mxc_s256", 256, 2, [0, 256], seed=321),
    make_workload("mxc_ragged", 700, 3, [0, 300, 700], seed=322, k_offset_var=2.0),
    make_workload("mxc_varlen", 1200, 2, [0, 0, 1, 64, 65, 193, 700, 700, 1200], seed=323),
]


@pytest.mark.parametrize("q_centre", [True, False])
@pytest.mark.parametrize("w", CAUSAL_CASES, ids=lambda w: w.name)
def test_mxfp4_causal_every_element(w, q_centre):
    """Causal FP4 plans (reading 8 of the FP4 reference): every element against
    its causal FP4 computation, the causal LSE, and the pages' FP4 bar against
    the float64 causal softmax."""
    plan, ws, out, lse, (q, k, v), hs = _run(w, q_centre, causal=True, lse=True)
    z = M.quantize_mxfp4(q, k, v, w.cu_seqlens, w.softmax_scale, q_centre=q_centre)
    _check_codes(read_mx(plan, ws, hs), z)
    ops = M.dequantized_operands(z, w.cu_seqlens)
    ref = M.attention_from_operands(ops["Q"], ops["QM"], ops["K"], ops["V"], w.cu_seqlens, causal=True)
    o = out.float().cpu().numpy()
    assert np.isfinite(o).all()
    _check_output(o, ref, w.name)
    _check_lse(lse, z, list(w.cu_seqlens), hs, causal=True)
    ex = exact.attention(q, k, v, w.cu_seqlens, w.softmax_scale, causal=True).numpy()
    # the pages' FP4 bar on rows that see at least FEW_KEYS keys: with fewer,
    # the method itself can miss it (tests/test_oracle_mxfp4.py shows a
    # 36-key row of this varlen case doing so in the reference), and those
    # rows are held to the reference's FP4 computation above
    few = visible_keys(w.cu_seqlens, True) < FEW_KEYS
    assert np.all((np.abs(o - ex) <= 1.0 + 0.1 * np.abs(ex))[~few])
    rel = np.linalg.norm(o - ex) / np.linalg.norm(ex)
    log(f"  rel RMS vs float64 causal softmax: {rel:.4f}")
    assert rel < 0.35


def test_mxfp4_causal_full_size_sampled():
    """The causal FP4 plan at S=30272, 56 heads: sampled rows of two heads and
    their LSE against the reference."""
    w = WORKLOADS["s30272_h56_koffset"]
    heads = [0, w.heads - 1]
    plan, ws, out, lse, (q, k, v), hs = _run(w, True, heads, poison=False, causal=True, lse=True)
    z = M.quantize_mxfp4(q, k, v, w.cu_seqlens, w.softmax_scale, q_centre=True)
    rows = sample_rows(w.tokens, 48, seed=78, cu_seqlens=w.cu_seqlens)
    ref = M.attention_mxfp4_rows(z, w.cu_seqlens, rows, list(range(len(hs))), causal=True)
    o = out[rows][:, hs].float().cpu().numpy()
    _check_output(o, ref, "causal " + w.name)
    lref = M.lse_mxfp4_rows(z, w.cu_seqlens, rows, list(range(len(hs))), causal=True)
    got = lse.cpu().double().numpy()[hs][:, rows].T
    check_lse_values(got, lref, "causal full size")


@pytest.mark.parametrize("name", ["s4096_h56", "s30272_h56_koffset", "varlen_30272_h56"])
def test_mxfp4_full_size_sampled(name):
    """Full sizes in the launch configuration the bench times: codes of two heads
    bit for bit, and sampled rows of those heads against the reference."""
    w = WORKLOADS[name]
    heads = [0, w.heads - 1]
    plan, ws, out, (q, k, v), hs = _run(w, True, heads, poison=False)
    z = M.quantize_mxfp4(q, k, v, w.cu_seqlens, w.softmax_scale, q_centre=True)
    _check_codes(read_mx(plan, ws, hs), z)
    rows = sample_rows(w.tokens, 48, seed=77, cu_seqlens=w.cu_seqlens)
    ref = M.attention_mxfp4_rows(z, w.cu_seqlens, rows, list(range(len(hs))))
    o = out[rows][:, hs].float().cpu().numpy()
    _check_output(o, ref, name)
