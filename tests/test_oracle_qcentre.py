"""Pins of the E4M3 oracle's Q centring (oracle.quantize.centre_q,
quantize(..., q_centre=True), qcentre_operand).

The FlashInfer "minimax_h3_sm120_varlen_attention_nvfp4" page centres Q rows by
the mean of their 128-row block and adds the block-mean term qm . k back to the
scores.  Each pin below fixes one part of that without reusing the oracle's
code path:
* block means against ``math.fsum`` per (block, head, channel), blocks counted
  from each segment's start over ragged segment lengths (a wrong block size,
  origin or row count fails);
* a Q whose blocks hold equal rows: every centred value is 0, so every code is
  0, and the operand is the block mean itself, so the attention equals the
  float64 attention of Q (a dropped, misplaced or negated mean term fails);
* a per-block constant added to Q (all arithmetic exact) moves qm by exactly
  that constant and leaves every code and scale unchanged (centring by another
  block, by the segment mean or not at all fails);
* zero-mean blocks: the codes and scales equal those of the uncentred
  quantizer bit for bit;
* on Q with a per-channel offset, the centred recipe's error against the exact
  attention is well below the uncentred one's (the reason for the variant).
"""
import math
from fractions import Fraction

import numpy as np
import torch

from oracle import attention as A
from oracle import compare
from oracle import e4m3
from oracle import quantize as Qz
from workloads import generate, make_workload

SIGMA = 0.125


def _bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def _blocks(cu):
    out = []
    for a, b in zip(cu[:-1], cu[1:]):
        for r in range(a, b, 128):
            out.append((r, min(r + 128, b)))
    return out


def test_block_means_against_fsum_over_ragged_segments():
    cu = [0, 0, 1, 128, 257, 557, 685, 685, 1000]
    rng = np.random.default_rng(11)
    q = _bf16(rng.normal(size=(cu[-1], 2, 8)) * 3.0)
    _, qm = Qz.centre_q(q, cu)
    blocks = _blocks(cu)
    assert qm.shape == (len(blocks), 2, 8)
    for i, (a, b) in enumerate(blocks):
        for h in range(2):
            for d in range(8):
                exact = Fraction(math.fsum(float(x) for x in q[a:b, h, d])) / (b - a)
                assert qm[i, h, d] == np.float32(float(exact)), (i, h, d)


def test_equal_rows_give_zero_codes_and_the_attention_of_q():
    cu = [0, 200, 200, 456, 521]
    T, H, D = cu[-1], 2, 16
    rng = np.random.default_rng(12)
    q = np.zeros((T, H, D), np.float32)
    for a, b in _blocks(cu):
        q[a:b] = _bf16(rng.normal(size=(H, D)) * 2.0)[None]
    k = _bf16(rng.normal(size=(T, H, D)))
    v = _bf16(rng.normal(size=(T, H, D)))
    r = Qz.quantize(q, k, v, cu, SIGMA, q_centre=True)
    assert not r["q_codes"].any()
    qop = Qz.qcentre_operand(r["q_codes"], r["scales"][0], r["qm"], cu)
    assert np.array_equal(qop, q.astype(np.float64))
    dk = Qz.dequantize(r["k_codes"], r["scales"][1])
    dv = Qz.dequantize(r["v_codes"], r["scales"][2])
    got = A.attention(qop, dk, dv, cu, SIGMA).numpy()
    ref = A.attention(q, dk, dv, cu, SIGMA).numpy()
    assert np.abs(got - ref).max() <= 1e-12


def test_per_block_constant_moves_the_mean_and_keeps_the_codes():
    cu = [0, 256, 256, 640, 1024]        # full 128-row blocks: every mean is exact
    T, H, D = cu[-1], 3, 8
    rng = np.random.default_rng(13)
    q = rng.integers(-64, 65, size=(T, H, D)).astype(np.float32) / 16.0
    k = _bf16(rng.normal(size=(T, H, D)))
    v = _bf16(rng.normal(size=(T, H, D)))
    blocks = _blocks(cu)
    shift = rng.integers(-40, 41, size=(len(blocks), H, D)).astype(np.float32) / 16.0
    q2 = q.copy()
    for i, (a, b) in enumerate(blocks):
        q2[a:b] += shift[i][None]
    r1 = Qz.quantize(q, k, v, cu, SIGMA, q_centre=True)
    r2 = Qz.quantize(q2, k, v, cu, SIGMA, q_centre=True)
    assert np.array_equal(r2["qm"], r1["qm"] + shift)
    assert np.array_equal(r2["q_codes"], r1["q_codes"])
    assert np.array_equal(r2["scales"], r1["scales"])
    # and without centring the codes do change
    assert not np.array_equal(Qz.quantize(q2, k, v, cu, SIGMA)["q_codes"],
                              Qz.quantize(q, k, v, cu, SIGMA)["q_codes"])


def test_zero_mean_blocks_reproduce_the_uncentred_quantizer():
    cu = [0, 384, 640]
    T, H, D = cu[-1], 2, 16
    rng = np.random.default_rng(14)
    q = np.zeros((T, H, D), np.float32)
    for a, b in _blocks(cu):
        half = _bf16(rng.normal(size=(64, H, D)) * 1.5)
        q[a:a + 64] = half
        q[a + 64:b] = -half
    k = _bf16(rng.normal(size=(T, H, D)))
    v = _bf16(rng.normal(size=(T, H, D)))
    rc = Qz.quantize(q, k, v, cu, SIGMA, q_centre=True)
    rp = Qz.quantize(q, k, v, cu, SIGMA)
    assert not rc["qm"].any()
    for name in ("q_codes", "k_codes", "v_codes", "scales", "mu"):
        assert np.array_equal(rc[name], rp[name]), name


def test_segment_scales_centre_each_segment_alone():
    cu = [0, 130, 130, 400]
    T, H, D = cu[-1], 2, 8
    rng = np.random.default_rng(15)
    q = _bf16(rng.normal(size=(T, H, D)) + 2.0)
    k = _bf16(rng.normal(size=(T, H, D)))
    v = _bf16(rng.normal(size=(T, H, D)))
    r = Qz.quantize_segments(q, k, v, cu, SIGMA, q_centre=True)
    whole = Qz.quantize(q, k, v, cu, SIGMA, q_centre=True)
    assert np.array_equal(r["qm"], whole["qm"])          # blocks never cross a segment
    for s, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        if b > a:
            one = Qz.quantize(q[a:b], k[a:b], v[a:b], [0, b - a], SIGMA, q_centre=True)
            assert np.array_equal(r["q_codes"][a:b], one["q_codes"])
            assert np.array_equal(r["scales"][:, s], one["scales"])
    qop = Qz.qcentre_operand(r["q_codes"], r["scales"][0], r["qm"], cu)
    assert qop.shape == (T, H, D)


def q_offset_case(T=2048, H=2, seed=77):
    """N(0, 1) inputs with per-(head, channel) offsets of variance 2 on K and on Q."""
    w = make_workload("q_offset", T, H, [0, T], seed=seed, k_offset_var=2.0, q_offset_var=2.0)
    return w, generate(w)


def test_centring_cuts_the_error_on_offset_q():
    w, (q, k, v) = q_offset_case()
    cu = w.cu_seqlens
    ref = A.attention(q, k, v, cu, w.softmax_scale).numpy()
    rows = list(range(0, w.tokens, 8))

    def err(r, qop):
        dk = Qz.dequantize(r["k_codes"], r["scales"][1])
        dv = Qz.dequantize(r["v_codes"], r["scales"][2])
        o = A.attention_fp8_recipe(qop, dk, dv, cu, w.softmax_scale, rows=rows).numpy()
        return compare.rel_rms(o, ref[rows])

    rp = Qz.quantize(q, k, v, cu, w.softmax_scale)
    rc = Qz.quantize(q, k, v, cu, w.softmax_scale, q_centre=True)
    plain = err(rp, Qz.dequantize(rp["q_codes"], rp["scales"][0]))
    centred = err(rc, Qz.qcentre_operand(rc["q_codes"], rc["scales"][0], rc["qm"], cu))
    assert centred <= 0.92 * plain, (centred, plain)
    # the centred codes use E4M3's range on the centred values only
    assert e4m3.decode(rc["q_codes"]).max() <= 448.0
