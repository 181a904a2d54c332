"""Planted mistakes in the oracle must fail its pins.

Every oracle function is pinned by checks that do not reuse its code path
(brute force, closed forms, invariants, lossless special cases).  This file
checks that the pins are strong enough: each mutant below edits ONE
expression of ONE oracle function (a dropped term, a wrong sign, constant,
index, axis or operand), rebuilds that function from the edited source in the
oracle module's namespace, puts it in place for the duration of one test, and
runs the module's positive pins; at least one of them must fail.  Nothing is
changed on disk, and the GPU is not involved.

A mutant that no pin detects is a gap in the pins, not a passing test: the
assertion names it.
"""
import inspect
import itertools
import textwrap

import pytest

from oracle import attention as A
from oracle import e4m3 as E
from oracle import mxfp4 as M
from oracle import quantize as Qz
from tests import test_oracle_attention as TA
from tests import test_oracle_e4m3 as TE
from tests import test_oracle_fp8_recipe as TF
from tests import test_oracle_mxfp4 as TM
from tests import test_oracle_qcentre as TQC
from tests import test_oracle_quantize as TQ


def _mutant(mod, fname, old, new):
    """``mod.fname`` rebuilt from its source with ``old`` replaced by ``new``
    (``old`` must occur exactly once)."""
    src = textwrap.dedent(inspect.getsource(getattr(mod, fname)))
    assert src.count(old) == 1, f"{fname}: {old!r} occurs {src.count(old)} times"
    ns = {}
    exec(compile(src.replace(old, new), f"<mutant of {mod.__name__}.{fname}>", "exec"), mod.__dict__, ns)
    return ns[fname]


def _param_sets(fn):
    """Argument dicts for a test function from its parametrize marks (one empty dict if none)."""
    marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    if not marks:
        return [{}]
    per_mark = []
    for m in marks:
        names = [n.strip() for n in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
        sets = []
        for vals in m.args[1]:
            vals = getattr(vals, "values", vals)            # pytest.param(...)
            if len(names) == 1:
                vals = (vals,) if not (isinstance(vals, tuple) and len(vals) == 1) else vals
            sets.append(dict(zip(names, vals)))
        per_mark.append(sets)
    return [dict(itertools.chain.from_iterable(d.items() for d in combo)) for combo in itertools.product(*per_mark)]


def _failures(test_module, names):
    """Run the named pins of ``test_module`` (every parameter set); return the failing ones."""
    failed = []
    for name in names:
        fn = getattr(test_module, name)
        for kwargs in _param_sets(fn):
            try:
                fn(**kwargs)
            except Exception as exc:                        # an AssertionError, or the mutant crashing the pin
                failed.append(f"{name}{kwargs or ''}: {type(exc).__name__}")
    return failed


ATTENTION_PINS = ["test_brute_force_mpmath", "test_rows_api_matches_full", "test_one_hot_returns_v_row_exactly",
                  "test_equal_scores_give_mean_of_v", "test_length_one_segment_returns_v",
                  "test_segment_independence", "test_k_shift_invariance", "test_permutation_equivariance",
                  "test_lse_rows_closed_form", "test_causal_brute_force_mpmath",
                  "test_causal_row_equals_prefix_segment", "test_lse_rows_two_keys_closed_form",
                  "test_lse_rows_brute_force_mpmath"]
QUANTIZE_PINS = ["test_plain_scale_closed_form_and_codes", "test_mean_equals_exact_rational_mean",
                 "test_mean_fixed_chunk_order", "test_k_amax_min_max_route_and_mu_layout",
                 "test_k_shift_leaves_codes_unchanged_when_mean_is_exact", "test_quantize_bundle_shapes",
                 "test_q_scale_pow2_properties", "test_q_scale_pow2_worked_cases",
                 "test_quantize_with_softmax_scale_changes_only_q", "test_segment_scales_single_segment_is_per_head",
                 "test_segment_scales_are_independent_of_other_segments",
                 "test_segment_scales_power_of_two_rescaling", "test_q_scale_pow2_bits_match_exact_arithmetic",
                 "test_q_scale_pow2_bits_where_t_is_a_power_of_two"]
E4M3_PINS = ["test_exhaustive_bf16_against_brute_force", "test_dense_float32_grid_against_brute_force",
             "test_matches_torch_float8_e4m3fn_cast", "test_golden_worked_values", "test_nan_and_inf",
             "test_decode_roundtrip_every_code"]
RECIPE_PINS = ["test_equal_scores_give_mean_of_v", "test_one_dominant_key_returns_its_v_row",
               "test_powers_of_two_probabilities_are_exact", "test_rows_api_matches_full"]
MXFP4_PINS = ["test_e2m1_table_against_ocp_values", "test_e2m1_encode_brute_force", "test_block_exp_brute_force",
              "test_mx_quantize_error_bound_and_range", "test_quantize_probs_closed_forms",
              "test_one_hot_key_returns_its_value_row", "test_equal_scores_return_mean_of_v",
              "test_lossless_inputs_reduce_to_plain_softmax", "test_segments_and_q_blocks_are_independent",
              "test_block_mean_centring_identical_rows", "test_causal_lossless_inputs_reduce_to_plain_causal_softmax",
              "test_lse_lossless_inputs_equal_the_float64_lse", "test_q_block_means_equal_exact_rational_means",
              "test_lse_is_the_log_of_the_quantized_weights"]
QCENTRE_PINS = ["test_block_means_against_fsum_over_ragged_segments",
                "test_equal_rows_give_zero_codes_and_the_attention_of_q",
                "test_per_block_constant_moves_the_mean_and_keeps_the_codes",
                "test_zero_mean_blocks_reproduce_the_uncentred_quantizer",
                "test_segment_scales_centre_each_segment_alone", "test_centring_cuts_the_error_on_offset_q"]

# (oracle module, function, expression, planted replacement, pins module, pin names, what the mistake is)
MUTANTS = [
    # float64 attention (the definition on the FlashInfer page)
    (A, "_segment_rows", "s = torch.matmul(qh, kh) * sigma", "s = torch.matmul(qh, kh)", TA, ATTENTION_PINS,
     "softmax scale dropped"),
    (A, "_segment_rows", "s = torch.matmul(qh, kh) * sigma", "s = torch.matmul(qh, kh) * sigma * sigma", TA,
     ATTENTION_PINS, "softmax scale applied twice"),
    (A, "_segment_rows", "s = torch.matmul(qh, kh) * sigma", "s = -torch.matmul(qh, kh) * sigma", TA,
     ATTENTION_PINS, "score sign flipped"),
    (A, "_segment_rows", "kh = ks.permute(1, 2, 0)", "kh = vs.permute(1, 2, 0)", TA, ATTENTION_PINS,
     "V used as the key operand"),
    (A, "_segment_rows", "vh = vs.permute(1, 0, 2)", "vh = ks.permute(1, 0, 2)", TA, ATTENTION_PINS,
     "K used as the value operand"),
    (A, "_segment_rows", "o = torch.matmul(p, vh) / l", "o = torch.matmul(p, vh)", TA, ATTENTION_PINS,
     "softmax not normalized"),
    (A, "_segment_rows", "l = p.sum(dim=-1, keepdim=True)", "l = p.sum(dim=-2, keepdim=True)", TA,
     ATTENTION_PINS, "normalizer summed over the query axis"),
    (A, "_segment_rows", "p = torch.exp(s - m)", "p = torch.exp(2 * (s - m))", TA, ATTENTION_PINS,
     "exponential of twice the score (log2 and ln mixed up)"),
    (A, "_causal_mask", "torch.arange(L)[None, :] > torch", "torch.arange(L)[None, :] >= torch", TA,
     ATTENTION_PINS, "causal query does not see itself"),
    (A, "attention", "kd[a:b], vd[a:b]", "kd[a:], vd[a:]", TA, ATTENTION_PINS,
     "keys run past the segment end"),
    (A, "attention_rows", "kd[a:b], vd[a:b]", "kd[:b], vd[:b]", TA, ATTENTION_PINS,
     "keys start before the segment start"),
    (A, "lse_rows", "kd[a:kend]) * sigma", "kd[a:kend])", TA, ATTENTION_PINS, "LSE without the softmax scale"),
    (A, "lse_rows", "torch.logsumexp(sc, dim=-1)", "torch.logsumexp(sc, dim=-1) - math.log(sc.shape[-1])",
     TA, ATTENTION_PINS, "log-mean-exp instead of log-sum-exp"),
    (A, "lse_rows", "kend = r + 1 if causal else b", "kend = r + 2 if causal else b", TA, ATTENTION_PINS,
     "causal LSE sees the next key"),
    # the FP8 recipe (sglang FP8 PR, "Modifications")
    (A, "attention_fp8_recipe", "kd[a:kend]) * sigma", "kd[a:kend])", TF, RECIPE_PINS,
     "recipe without the softmax scale"),
    (A, "attention_fp8_recipe", "/ ph.sum(dim=-1, keepdim=True)", "/ ph.sum(dim=0, keepdim=True)", TF,
     RECIPE_PINS, "recipe normalized over the wrong axis"),
    (A, "attention_fp8_recipe", 'torch.einsum("hl,lhd->hd", ph, vd[a:kend])',
     'torch.einsum("hl,lhd->hd", ph, kd[a:kend])', TF, RECIPE_PINS, "recipe weights K instead of V"),
    (A, "attention_fp8_recipe", "kend = r + 1 if causal else b", "kend = r if causal else b", TF, RECIPE_PINS,
     "causal recipe misses the query's own key"),
    # E4M3 encoder / decoder (OCP OFP8 E4M3)
    (E, "_encode", "e = e2.astype(np.int64) - 1", "e = e2.astype(np.int64)", TE, E4M3_PINS,
     "exponent off by one"),
    (E, "_encode", "normal = (e + 7) * 8", "normal = (e + 8) * 8", TE, E4M3_PINS, "exponent bias 8"),
    (E, "_encode", "np.round(frac8)", "np.floor(frac8)", TE, E4M3_PINS, "mantissa truncated"),
    (E, "_encode", "np.round(frac8)", "np.floor(frac8 + 0.5)", TE, E4M3_PINS, "ties rounded up, not to even"),
    (E, "_encode", "(mag <= 0x7E), mag, 0x7E)", "(mag <= 0x7F), mag, 0x7F)", TE, E4M3_PINS,
     "no saturation at 448"),
    (E, "_encode", "sub = np.round(a * 2.0 ** 9)", "sub = np.round(a * 2.0 ** 10)", TE, E4M3_PINS,
     "subnormal step 2^-10"),
    (E, "decode", "np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)", TE, E4M3_PINS,
     "decoder bias 8"),
    (E, "decode", "(1.0 + m / 8.0)", "(1.0 + m / 16.0)", TE, E4M3_PINS, "decoder mantissa in sixteenths"),
    (E, "decode", "m * 2.0 ** -9", "m * 2.0 ** -10", TE, E4M3_PINS, "decoder subnormal step"),
    # per-head quantizer (amax / 448, K centred by its segment mean)
    (Qz, "head_scale", "amax / np.float32(448.0)", "amax / np.float32(240.0)", TQ, QUANTIZE_PINS,
     "scale from 240 instead of 448"),
    (Qz, "head_scale", "np.where(amax == 0, np.float32(1.0), s)", "s", TQ, QUANTIZE_PINS,
     "all-zero head gets scale 0"),
    (Qz, "segment_mean", "(total / float(b - a))", "(total / float(b - a + 1))", TQ, QUANTIZE_PINS,
     "mean divided by L + 1"),
    (Qz, "segment_mean", "for t in range(c, min(c + CHUNK, b)):", "for t in range(c + 1, min(c + CHUNK, b)):",
     TQ, QUANTIZE_PINS, "first row of every chunk dropped from the mean"),
    (Qz, "quantize_k", "y[a:b] = xf[a:b] - mu[s][None]", "y[a:b] = xf[a:b] + mu[s][None]", TQ, QUANTIZE_PINS,
     "K mean added instead of subtracted"),
    (Qz, "quantize_k", "y[a:b] = xf[a:b] - mu[s][None]", "y[a:b] = xf[a:b]", TQ, QUANTIZE_PINS,
     "K not centred"),
    (Qz, "quantize_plain", "np.abs(xf).max(axis=(0, 2))", "xf.max(axis=(0, 2))", TQ, QUANTIZE_PINS,
     "amax without the absolute value"),
    (Qz, "encode_at_scale", "_as_f32(x) / np.asarray(s, np.float32)", "_as_f32(x) * np.asarray(s, np.float32)",
     TQ, QUANTIZE_PINS, "codes of x times the scale"),
    (Qz, "q_scale_pow2", "m = int(e) - 1 if fr == 0.5 else int(e)", "m = int(e)", TQ, QUANTIZE_PINS,
     "Q scale doubled when the product is already a power of two"),
    (Qz, "q_scale_pow2", "f = (np.float32(softmax_scale) * s_k) * LOG2E_F32", "f = np.float32(softmax_scale) * s_k",
     TQ, QUANTIZE_PINS, "score factor without log2(e)"),
    (Qz, "quantize", 'q_scale_pow2(rq["scale"], rk["scale"], softmax_scale)',
     'q_scale_pow2(rq["scale"], rq["scale"], softmax_scale)', TQ, QUANTIZE_PINS,
     "Q's power-of-two rule fed Q's scale instead of K's"),
    # block-scaled FP4 variant (MX form of the NVFP4 recipe on the FlashInfer page)
    (M, "e2m1_encode", "mag = np.minimum(mag, 7)", "mag = np.minimum(mag, 6)", TM, MXFP4_PINS,
     "E2M1 saturating at 4"),
    (M, "e2m1_encode", "np.round(half_units)", "np.floor(half_units)", TM, MXFP4_PINS, "E2M1 mantissa truncated"),
    (M, "block_exp", "out[i] = min(max(e, -127), 127)", "out[i] = min(max(e + 1, -127), 127)", TM, MXFP4_PINS,
     "block exponent one too large"),
    (M, "quantize_probs", "np.ceil(xb.max(axis=-1, keepdims=True) - LOG2_6)",
     "np.floor(xb.max(axis=-1, keepdims=True) - LOG2_6)", TM, MXFP4_PINS, "P block scale rounded down"),
    (M, "attention_from_operands", "x = Q[a:b, h] @ Kh.T + QM[a:b, h] @ Kh.T", "x = Q[a:b, h] @ Kh.T", TM,
     MXFP4_PINS, "block-mean term dropped"),
    (M, "attention_from_operands", "out[a:b, h] = (p @ V[a:b, h])", "out[a:b, h] = (p.T @ V[a:b, h])", TM,
     MXFP4_PINS, "P transposed"),
    (M, "quantize_mxfp4", "qy[a:b] = (qf[a:b] - qm[i][None]) * c", "qy[a:b] = (qf[a:b] + qm[i][None]) * c", TM,
     MXFP4_PINS, "Q block mean added instead of subtracted"),
    (M, "block_mean", "(total / float(b - a))", "(total / float(QBLOCK))", TM, MXFP4_PINS,
     "short last Q block divided by 128"),
    (M, "score_factor", "np.float32(softmax_scale) * LOG2E_F32", "np.float32(softmax_scale)", TM, MXFP4_PINS,
     "FP4 score factor without log2(e)"),
    # E4M3 Q centring
    (Qz, "centre_q", "qc[a:b] = qf[a:b] - qm[i][None]", "qc[a:b] = qf[a:b] + qm[i][None]", TQC, QCENTRE_PINS,
     "E4M3 Q block mean added instead of subtracted"),
    (Qz, "centre_q", "qc[a:b] = qf[a:b] - qm[i][None]", "qc[a:b] = qf[a:b]", TQC, QCENTRE_PINS,
     "E4M3 Q not centred"),
    (Qz, "centre_q", "qm[i] = block_mean(qf, a, b)", "qm[i] = block_mean(qf, a, min(b, a + 64))", TQC,
     QCENTRE_PINS, "E4M3 Q mean over 64 rows of the block"),
    (Qz, "qcentre_operand", "+ np.asarray(qm[i], np.float64)[None]", "- np.asarray(qm[i], np.float64)[None]", TQC,
     QCENTRE_PINS, "mean term subtracted from the Q operand"),
    (Qz, "qcentre_operand", "+ np.asarray(qm[i], np.float64)[None]", "+ 0.0", TQC, QCENTRE_PINS,
     "mean term dropped from the Q operand"),
    (Qz, "qcentre_operand", "+ np.asarray(qm[i], np.float64)[None]", "+ np.asarray(qm[max(i - 1, 0)], np.float64)[None]",
     TQC, QCENTRE_PINS, "mean term of the previous block"),
]


@pytest.mark.filterwarnings("ignore::RuntimeWarning")   # some mutants divide by zero on purpose
@pytest.mark.parametrize("mod,fname,old,new,tmod,pins,what", MUTANTS, ids=[m[-1] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(monkeypatch, mod, fname, old, new, tmod, pins, what):
    monkeypatch.setattr(mod, fname, _mutant(mod, fname, old, new))
    failed = _failures(tmod, pins)
    assert failed, f"no pin of {tmod.__name__} detects the planted mistake: {what} ({fname})"


def test_unmutated_oracle_passes_every_pin_run_here():
    """The harness itself: with no mutant in place every pin listed above passes."""
    for tmod, pins in ((TA, ATTENTION_PINS), (TF, RECIPE_PINS), (TE, E4M3_PINS), (TQ, QUANTIZE_PINS),
                       (TM, MXFP4_PINS), (TQC, QCENTRE_PINS)):
        assert _failures(tmod, pins) == []
