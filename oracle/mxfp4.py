"""CPU reference for the block-scaled FP4 variant of the attention (MXFP4
operands and probabilities).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the product path.

What it follows (FlashInfer "minimax_h3_sm120_varlen_attention_nvfp4" page,
the description of the kernel under the output formula):

* The output is still ``softmax(q k^T softmax_scale) v`` per segment and head;
  only the operands of both products are block-scaled FP4.
* K rows are centred by the segment's per-channel mean (as in the E4M3 path,
  ``quantize.segment_mean``), Q rows by the mean of their 128-row block, and
  the block-mean term ``qm . k`` is added back to the scores, so the softmax
  is that of the uncentred Q.
* Q, K and V are E2M1 codes with one scale per block of elements along the
  contraction axis (channels for Q and K, keys for the transposed V); the
  probabilities are E2M1 codes with one scale per block of keys, after the
  exponent has been taken against a per-query reference.
* The output is rounded to BF16 once (by the kernel; this module returns
  float64).

Readings (the page is written for SM120's NVFP4: UE4M3 scales on 16-element
blocks; gfx950's scaled matrix products take the OCP MX form, one E8M0
power-of-two scale per 32 elements, and this variant is built on that):

1. Block = 32 consecutive elements along the contraction axis.  Q and K:
   channels [32j, 32j+32) of a row.  V: keys [32b, 32b+32) of a segment
   (counted from the segment start) for one channel.  Probabilities: the same
   key blocks, for one query.  The Q mean block: rows [128i, 128i+128) of a
   segment (the last one may be shorter).
2. Block scale 2^e with e the smallest integer for which amax <= 6 * 2^e (the
   page's amax/6 rounded up to a power of two, so nothing clips); e = -127 for
   an all-zero block; e is kept in [-127, 127], the E8M0 range.
3. Codes: E2M1 of x / 2^e, round to nearest with ties to the even code,
   magnitudes above 6 saturate (only reachable at the clamp of reading 2).
   E2M1 (OCP MX): sign, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes
   0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7, code | 8 is the negative.
4. The score factor c = fl32(fl32(softmax_scale) * fl32(log2 e)) is folded
   into Q before quantization, so scores come out in log2 units:
   Q operand y = fl32(fl32(q - qm) * c) and block-mean operand fl32(qm * c),
   each quantized as in 2-3.  The block mean qm is a fixed-order float64 sum
   over the block's rows (ascending) divided by the row count, rounded to
   float32.  Without Q centring qm = 0 (y = fl32(q * c)).
5. Scores x_ij = sum_d Qhat_id Khat_jd + sum_d QMhat_d Khat_jd with the
   dequantized operands, in float64.
6. Probabilities (page: the two-level scheme whose first level only brings the
   row maximum into the UE4M3 scale's range; a power-of-two scale needs no
   such level): for query i and key block b, E = ceil(max_{j in b} x_ij -
   log2 6) and phat_ij = 2^E * e2m1(2^(x_ij - E)).  phat depends on x alone, not
   on any running reference (the kernel's references are whole powers of two).
7. out_i = sum_j phat_ij Vhat_j / sum_j phat_ij.
8. Causal (``causal=True``; the E4M3 path's reading): query i of a segment
   sees the keys j <= i of it; its probability blocks are the key blocks of
   reading 1 cut at the last visible key (the last block holds the visible
   keys only).
9. LSE (``lse_mxfp4_rows``): the natural-log log-sum-exp of the uncentred
   scores over the row's visible keys, taken (as for the E4M3 path) as the
   log of the row's normalizer, the sum of the weights phat of reading 6:
   ln 2 * (log2 sum_j phat_ij + (Qhat_i + QMhat_i) . mu), the second term
   adding back what centring K by its segment mean mu took out.  Where every
   weight is exact (phat = 2^x) this is the log-sum-exp itself.

Parity pins live in ``tests/test_oracle_mxfp4.py``.
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np

from .quantize import _as_f32, segment_mean, LOG2E_F32

BLOCK = 32          # elements per scale block
QBLOCK = 128        # Q rows per mean block
E2M1_MAX = 6.0
LOG2_6 = float(np.log2(6.0))
_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(code) -> np.ndarray:
    """float64 value of E2M1 codes 0..15."""
    c = np.asarray(code).astype(np.int64)
    mag = _GRID[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_encode(y) -> np.ndarray:
    """E2M1 codes (uint8, 0..15) of finite float values: round to nearest, ties
    to the even code, saturating at +-6; -0.0 keeps its sign (code 8)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    sign = np.signbit(y).astype(np.int64) << 3
    # normal range a >= 1: a = f * 2^E with f in [1, 2); mantissa in halves
    f2, e2 = np.frexp(np.clip(a, 1.0, 16.0))       # a = f2 * 2^e2, f2 in [0.5, 1); >= 16 saturates anyway
    E = e2.astype(np.int64) - 1
    half_units = (2.0 * f2 - 1.0) * 2.0            # 0 or 1 (or between), exact
    normal = (E + 1) * 2 + np.round(half_units).astype(np.int64)   # carry into the exponent is automatic
    sub = np.round(np.minimum(a, 1.0) * 2.0).astype(np.int64)   # a < 1: multiples of 0.5 (code 2 is 1.0)
    mag = np.where(a < 1.0, sub, normal)
    mag = np.minimum(mag, 7)
    return (mag | sign).astype(np.uint8)


def block_exp(amax, vmax: float = E2M1_MAX) -> np.ndarray:
    """Smallest integer e with amax <= vmax * 2^e (int64), -127 for amax == 0,
    clamped to [-127, 127].  Exact: the comparisons are between float64
    values that are exact (amax is a float32, vmax * 2^e a scaled small
    integer)."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.full(amax.shape, -127, np.int64)
    for i in np.ndindex(amax.shape):
        a = float(amax[i])
        if a == 0.0:
            continue
        e = int(np.ceil(np.log2(a / vmax)))
        while a > vmax * 2.0 ** e:
            e += 1
        while a <= vmax * 2.0 ** (e - 1):
            e -= 1
        out[i] = min(max(e, -127), 127)
    return out


def mx_quantize(y: np.ndarray, axis: int) -> Dict[str, np.ndarray]:
    """Block-scaled E2M1 quantization of float32 ``y`` along ``axis`` (its
    length a multiple of 32): codes (same shape, uint8 0..15) and e (the axis
    shortened by 32x, int64)."""
    y = np.asarray(y, np.float32)
    ym = np.moveaxis(y, axis, -1)
    n = ym.shape[-1]
    assert n % BLOCK == 0
    blocks = ym.reshape(ym.shape[:-1] + (n // BLOCK, BLOCK))
    e = block_exp(np.abs(blocks).max(axis=-1) if blocks.size else np.zeros(blocks.shape[:-1]))
    scaled = blocks.astype(np.float64) * np.ldexp(1.0, -e)[..., None]    # exact: power-of-two scaling
    codes = e2m1_encode(scaled).reshape(ym.shape)
    return {"codes": np.moveaxis(codes, -1, axis), "e": np.moveaxis(e, -1, axis) if e.ndim else e}


def mx_dequantize(codes: np.ndarray, e: np.ndarray, axis: int) -> np.ndarray:
    """float64 values of block-scaled codes (inverse layout of ``mx_quantize``)."""
    cm = np.moveaxis(np.asarray(codes), axis, -1)
    em = np.moveaxis(np.asarray(e), axis, -1)
    v = e2m1_decode(cm).reshape(cm.shape[:-1] + (cm.shape[-1] // BLOCK, BLOCK))
    v = v * np.ldexp(1.0, em.astype(np.int64))[..., None]
    return np.moveaxis(v.reshape(cm.shape), -1, axis)


def score_factor(softmax_scale: float) -> np.float32:
    """c = fl32(fl32(softmax_scale) * fl32(log2 e))."""
    return np.float32(np.float32(softmax_scale) * LOG2E_F32)


def q_blocks(cu_seqlens: Sequence[int]) -> List[tuple]:
    """(segment, first row, end row) of every 128-row Q block, in segment order."""
    out = []
    for s in range(len(cu_seqlens) - 1):
        a, b = cu_seqlens[s], cu_seqlens[s + 1]
        for r in range(a, b, QBLOCK):
            out.append((s, r, min(r + QBLOCK, b)))
    return out


def v_blocks(cu_seqlens: Sequence[int]) -> List[tuple]:
    """(segment, first key, end key) of every 32-key block, in segment order."""
    out = []
    for s in range(len(cu_seqlens) - 1):
        a, b = cu_seqlens[s], cu_seqlens[s + 1]
        for r in range(a, b, BLOCK):
            out.append((s, r, min(r + BLOCK, b)))
    return out


def block_mean(x: np.ndarray, a: int, b: int) -> np.ndarray:
    """Mean of rows [a, b) of x [T, H, D]: float64 sum in ascending row order,
    divided by the row count, rounded to float32."""
    total = np.zeros(x.shape[1:], np.float64)
    for t in range(a, b):
        total = total + x[t].astype(np.float64)
    return (total / float(b - a)).astype(np.float32)


def quantize_mxfp4(q, k, v, cu_seqlens: Sequence[int], softmax_scale: float,
                   q_centre: bool = True) -> Dict[str, np.ndarray]:
    """All operands of the FP4 variant.

    Returns (T tokens, H heads, D = 128 channels, nq Q blocks, nv V blocks):
      q_codes, k_codes, v_codes [T, H, D] uint8 (E2M1 codes, one per element);
      q_e, k_e [T, H, 4] (block exponents along channels);
      v_e [nv, H, D] (block exponents along keys, blocks of ``v_blocks``);
      qm [nq, H, D] float32 (block means, zero without centring);
      qm_codes [nq, H, D], qm_e [nq, H, 4] (the quantized fl32(qm * c));
      mu [nseg, H, D] float32 (K segment means); c (the score factor).
    """
    qf, kf, vf = _as_f32(q), _as_f32(k), _as_f32(v)
    T, H, D = qf.shape
    cu = list(cu_seqlens)
    nseg = len(cu) - 1
    c = score_factor(softmax_scale)

    mu = np.zeros((nseg, H, D), np.float32)
    ky = np.zeros_like(kf)
    for s in range(nseg):
        a, b = cu[s], cu[s + 1]
        if b > a:
            mu[s] = segment_mean(kf, a, b)
            ky[a:b] = kf[a:b] - mu[s][None]                  # float32, correctly rounded

    qb = q_blocks(cu)
    qm = np.zeros((len(qb), H, D), np.float32)
    qy = np.zeros_like(qf)
    for i, (s, a, b) in enumerate(qb):
        if q_centre:
            qm[i] = block_mean(qf, a, b)
        qy[a:b] = (qf[a:b] - qm[i][None]) * c                # two float32 roundings, in this order
    qmc = (qm * c).astype(np.float32)

    vb = v_blocks(cu)
    v_codes = np.zeros((T, H, D), np.uint8)
    v_e = np.zeros((len(vb), H, D), np.int64)
    for i, (s, a, b) in enumerate(vb):
        blk = np.zeros((BLOCK, H, D), np.float32)
        blk[: b - a] = vf[a:b]                               # a short last block is padded with zeros
        r = mx_quantize(blk, axis=0)
        v_codes[a:b] = r["codes"][: b - a]
        v_e[i] = r["e"][0]

    rq = mx_quantize(qy, axis=2)
    rk = mx_quantize(ky, axis=2)
    rm = mx_quantize(qmc, axis=2)
    return {"q_codes": rq["codes"], "q_e": rq["e"], "k_codes": rk["codes"], "k_e": rk["e"],
            "v_codes": v_codes, "v_e": v_e, "qm": qm, "qm_codes": rm["codes"], "qm_e": rm["e"],
            "mu": mu, "c": c}


def dequantized_operands(z: Dict[str, np.ndarray], cu_seqlens: Sequence[int]) -> Dict[str, np.ndarray]:
    """float64 operands: Q [T, H, D], K [T, H, D], V [T, H, D] and, per token,
    the block-mean operand of its Q block QM [T, H, D] (scores in log2 units)."""
    cu = list(cu_seqlens)
    Q = mx_dequantize(z["q_codes"], z["q_e"], axis=2)
    K = mx_dequantize(z["k_codes"], z["k_e"], axis=2)
    QMb = mx_dequantize(z["qm_codes"], z["qm_e"], axis=2)
    QM = np.zeros_like(Q)
    for i, (s, a, b) in enumerate(q_blocks(cu)):
        QM[a:b] = QMb[i][None]
    V = np.zeros(z["v_codes"].shape, np.float64)
    for i, (s, a, b) in enumerate(v_blocks(cu)):
        V[a:b] = e2m1_decode(z["v_codes"][a:b]) * np.ldexp(1.0, z["v_e"][i])[None]
    return {"Q": Q, "K": K, "V": V, "QM": QM}


def quantize_probs(x: np.ndarray) -> np.ndarray:
    """Reading 6: x [..., L] scores in log2 units of query rows -> phat [..., L]
    (float64), key blocks of 32 from the start of each row (a short last
    block holds the remaining keys)."""
    x = np.asarray(x, np.float64)
    L = x.shape[-1]
    nb = (L + BLOCK - 1) // BLOCK
    xp = np.full(x.shape[:-1] + (nb * BLOCK,), -np.inf)
    xp[..., :L] = x
    xb = xp.reshape(x.shape[:-1] + (nb, BLOCK))
    E = np.ceil(xb.max(axis=-1, keepdims=True) - LOG2_6)
    with np.errstate(invalid="ignore"):
        codes = e2m1_encode(np.exp2(xb - E))                # exp2(-inf) = 0 for the padding
    p = np.ldexp(e2m1_decode(codes), E.astype(np.int64))
    return p.reshape(xp.shape)[..., :L]


def attention_from_operands(Q, QM, K, V, cu_seqlens: Sequence[int], causal: bool = False) -> np.ndarray:
    """Readings 5-8 on dequantized float64 operands [T, H, D] (scores
    x = Q.K + QM.K in log2 units).  Returns float64 [T, H, D]."""
    Q, QM, K, V = (np.asarray(t, np.float64) for t in (Q, QM, K, V))
    T, H, D = Q.shape
    out = np.zeros((T, H, D), np.float64)
    cu = list(cu_seqlens)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b <= a:
            continue
        for h in range(H):
            Kh = K[a:b, h]                                   # [L, D]
            x = Q[a:b, h] @ Kh.T + QM[a:b, h] @ Kh.T         # [L, L]
            if causal:
                for i in range(b - a):                       # row i sees keys 0 .. i
                    p = quantize_probs(x[i, :i + 1])
                    out[a + i, h] = (p @ V[a:a + i + 1, h]) / p.sum()
                continue
            p = quantize_probs(x)
            out[a:b, h] = (p @ V[a:b, h]) / p.sum(axis=1, keepdims=True)
    return out


def attention_mxfp4(q, k, v, cu_seqlens: Sequence[int], softmax_scale: float,
                    q_centre: bool = True, causal: bool = False) -> np.ndarray:
    """The whole variant: quantize, then readings 5-8.  float64 [T, H, D]."""
    z = quantize_mxfp4(q, k, v, cu_seqlens, softmax_scale, q_centre)
    ops = dequantized_operands(z, cu_seqlens)
    return attention_from_operands(ops["Q"], ops["QM"], ops["K"], ops["V"], cu_seqlens, causal)


def _row_keys(cu: List[int], r: int, causal: bool):
    s = int(np.searchsorted(cu, r, side="right")) - 1
    return s, cu[s], (r + 1 if causal else cu[s + 1])


def attention_mxfp4_rows(z: Dict[str, np.ndarray], cu_seqlens: Sequence[int],
                         rows: Sequence[int], heads: Sequence[int], causal: bool = False) -> np.ndarray:
    """Selected output rows and heads of readings 5-8 from quantized operands
    ``z`` (each row against its own segment).  float64 [len(rows), len(heads), D]."""
    cu = list(cu_seqlens)
    ops = dequantized_operands(z, cu)
    out = np.zeros((len(rows), len(heads), ops["Q"].shape[2]), np.float64)
    for n, r in enumerate(rows):
        _, a, e = _row_keys(cu, r, causal)
        for m, h in enumerate(heads):
            Kh = ops["K"][a:e, h]
            x = Kh @ ops["Q"][r, h] + Kh @ ops["QM"][r, h]
            p = quantize_probs(x)
            out[n, m] = (p @ ops["V"][a:e, h]) / p.sum()
    return out


def lse_mxfp4_rows(z: Dict[str, np.ndarray], cu_seqlens: Sequence[int],
                   rows: Sequence[int], heads: Sequence[int], causal: bool = False) -> np.ndarray:
    """Reading 9: natural-log LSE of the uncentred scores per (row, head) from
    the dequantized operands of ``z``, as the log of the sum of the row's
    quantized weights.  float64 [len(rows), len(heads)]."""
    cu = list(cu_seqlens)
    ops = dequantized_operands(z, cu)
    out = np.zeros((len(rows), len(heads)), np.float64)
    for n, r in enumerate(rows):
        s, a, e = _row_keys(cu, r, causal)
        for m, h in enumerate(heads):
            qop = ops["Q"][r, h] + ops["QM"][r, h]
            x = ops["K"][a:e, h] @ qop
            lse2 = np.log2(np.sum(quantize_probs(x))) + qop @ z["mu"][s, h].astype(np.float64)
            out[n, m] = lse2 * np.log(2.0)
    return out
