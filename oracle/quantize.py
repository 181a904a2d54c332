"""CPU reference for the per-head E4M3 quantization of Q, K and V.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the product path.

What it follows
---------------
* Two passes per tensor, a per-head amax and then the pack into E4M3 codes
  (sglang PR "[diffusion] attention: add fp8_fa_sm120 FP8 backend for SM120
  GPUs", "Modifications", the fused_prep item).
* Scale ``s_h = fl32(amax_h / 448)`` per (tensor, head) over every token of the
  call, and ``1.0`` for an all-zero head (reading of "per-head scale =
  amax/448"; E4M3 max is 448).
* K is centred by its segment's per-channel mean before quantization.  The
  FlashInfer "minimax_h3_sm120_varlen_attention_nvfp4" page does this for its
  block-scaled operands and notes that the softmax is unchanged by it: a
  per-segment constant added to every key only adds a per-query constant to
  every score of that segment.  Q is not centred unless asked for (Q
  centring below).
* Codes: ``e4m3(fl32(y / s_h))`` with IEEE float32 division, where ``y = x``
  for Q and V and ``y = fl32(x - mu)`` for K.

Fixed-order mean (a reading; the pages fix no summation order): for segment
``[a, b)``, channel ``(h, d)``:

    sum64 = 0.0;  for each 256-token chunk [c, min(c+256, b)), c = a, a+256, ...
        chunk = 0.0;  for t in chunk, ascending:  chunk = chunk + x[t]   (float64)
        sum64 = sum64 + chunk                                             (float64)
    mu = fl32(fl64(sum64 / L))

Empty segments have no mean; their ``mu`` rows are 0.

Q's scale (``q_scale_pow2``): the pages ask for per-head amax scaling and fix
no exact formula.  The reading taken for Q is the smallest scale at or above
fl32(amax/448) that makes the score factor ``softmax_scale * s_q * s_k *
log2(e)`` a power of two, so the attention applies it exactly as a power-of-two
factor of the score products; K and V keep fl32(amax/448).  ``quantize`` uses
it when a ``softmax_scale`` is given and the plain amax/448 scale otherwise.
Parity pins live in ``tests/test_oracle_quantize.py``; for ``q_scale_pow2``:
its float32 bits against the same steps evaluated in exact rational
arithmetic with a search for the power of two (which catches an off-by-one in
the exponent where fl32(f * base) is itself a power of two), plus range
properties (at least amax/448, below twice it, factor a power of two).

Q centring (``centre_q``, ``quantize(..., q_centre=True)``): the FlashInfer
page centres Q rows by the mean of their 128-row block and adds the block-mean
term qm . k back to the scores, so the softmax is that of the uncentred Q.
The reading taken for E4M3 operands: Q's amax, scale and codes are those of
fl32(q - qm); the mean term is added back exactly (``qcentre_operand`` gives
the float64 operand dequant(code) * s_q + qm, which the attention oracle then
takes as its Q).  The block mean is the same fixed-order mean as the FP4
variant's (``mxfp4.block_mean`` over ``mxfp4.q_blocks``).  Pins: a Q whose
blocks hold equal rows gives all-zero codes and an output equal to the
float64 attention of the block means; adding a per-block constant to Q (all
values exact) shifts qm by that constant and leaves every code unchanged;
zero-mean blocks reproduce the uncentred quantization bit for bit; the block
means against ``math.fsum`` per block and channel.

Per-(segment, head) scales (``quantize_segments``) are a variant the product
offers for packed batches: the sglang PR quantizes per head over the whole
call, and a packed batch of unrelated sequences then shares one scale per
head; here each segment gets the per-head rule over its own tokens.  Pins:
a single segment reproduces ``quantize``; codes of a segment do not change
when another segment's values do; scaling one segment's tensor by a power of
two scales only that segment's scale by it and leaves every code unchanged.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np

from . import e4m3

CHUNK = 256


def _as_f32(x) -> np.ndarray:
    """BF16 tensor (torch) or array -> float32 numpy array (exact widening)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").float().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float32)


def head_scale(amax: np.ndarray) -> np.ndarray:
    """fl32(amax / 448) per head, 1.0 where amax == 0."""
    amax = np.asarray(amax, dtype=np.float32)
    s = amax / np.float32(448.0)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


LOG2E_F32 = np.float32(1.4426950408889634)


def q_scale_pow2(base: np.ndarray, s_k: np.ndarray, softmax_scale: float) -> np.ndarray:
    """Q's per-head scale: ``base`` (amax/448) rounded up to the smallest
    fl32(2^m / f), f = fl32(fl32(softmax_scale * s_k) * log2(e)), with
    2^m >= fl32(f * base); ``base`` itself where fl32(f * base) is not a normal
    float.  All arithmetic in float32, in the order written."""
    base = np.asarray(base, np.float32)
    s_k = np.asarray(s_k, np.float32)
    f = (np.float32(softmax_scale) * s_k) * LOG2E_F32
    t = (f * base).astype(np.float32)
    out = base.copy()
    for i in np.ndindex(t.shape):
        ti = np.float32(t[i])
        if not (np.float32(2.0 ** -126) <= ti < np.float32(2.0 ** 126)):
            continue
        fr, e = np.frexp(ti)                    # ti = fr * 2^e, fr in [0.5, 1)
        m = int(e) - 1 if fr == 0.5 else int(e)
        out[i] = np.float32(2.0 ** m) / np.float32(f[i])
    return out.astype(np.float32)


def segment_mean(x: np.ndarray, a: int, b: int) -> np.ndarray:
    """Fixed-order float64 mean of rows [a, b) of x [T, H, D], rounded to float32."""
    H, D = x.shape[1], x.shape[2]
    if b <= a:
        return np.zeros((H, D), np.float32)
    total = np.zeros((H, D), np.float64)
    for c in range(a, b, CHUNK):
        chunk = np.zeros((H, D), np.float64)
        for t in range(c, min(c + CHUNK, b)):
            chunk = chunk + x[t].astype(np.float64)
        total = total + chunk
    return (total / float(b - a)).astype(np.float32)


def encode_at_scale(x, s: np.ndarray) -> np.ndarray:
    """E4M3 codes of fl32(x / s_h): codes [T, H, D] uint8 for per-head scales s [H]."""
    y = _as_f32(x) / np.asarray(s, np.float32)[None, :, None]   # float32 / float32: IEEE division
    return e4m3.encode(y)


def quantize_plain(x, scale: np.ndarray = None) -> Dict[str, np.ndarray]:
    """Per-head quantization of Q or V: codes [T, H, D] uint8, scale [H] float32
    (amax/448 unless ``scale`` is given)."""
    xf = _as_f32(x)
    if scale is None:
        amax = np.abs(xf).max(axis=(0, 2)) if xf.shape[0] > 0 else np.zeros(xf.shape[1], np.float32)
        scale = head_scale(amax)
    s = np.asarray(scale, np.float32)
    return {"codes": encode_at_scale(xf, s), "scale": s}


def quantize_k(x, cu_seqlens: List[int]) -> Dict[str, np.ndarray]:
    """Per-head quantization of K after per-(segment, head, channel) centring.

    Returns codes [T, H, D] uint8, scale [H] float32, mu [nseg, H, D] float32.
    """
    xf = _as_f32(x)
    T, H, D = xf.shape
    nseg = len(cu_seqlens) - 1
    mu = np.zeros((nseg, H, D), np.float32)
    y = np.zeros_like(xf)
    for s in range(nseg):
        a, b = cu_seqlens[s], cu_seqlens[s + 1]
        mu[s] = segment_mean(xf, a, b)
        y[a:b] = xf[a:b] - mu[s][None]            # float32 subtraction, correctly rounded
    amax = np.abs(y).max(axis=(0, 2)) if T > 0 else np.zeros(H, np.float32)
    sc = head_scale(amax)
    codes = e4m3.encode(y / sc[None, :, None])
    return {"codes": codes, "scale": sc, "mu": mu}


def centre_q(q, cu_seqlens: List[int]):
    """Q centred by the mean of its 128-row block (Q centring of the FlashInfer
    page): returns (fl32(q - qm) [T, H, D] float32, qm [nq, H, D] float32) with
    qm the fixed-order mean of each block of ``mxfp4.q_blocks`` (segments in
    order, blocks of a segment counted from its start, the last one possibly
    shorter): a float64 sum over the block's rows in ascending order, divided
    by the row count, rounded to float32."""
    from .mxfp4 import block_mean, q_blocks
    qf = _as_f32(q)
    blocks = q_blocks(cu_seqlens)
    qm = np.zeros((len(blocks), qf.shape[1], qf.shape[2]), np.float32)
    qc = np.zeros_like(qf)
    for i, (_, a, b) in enumerate(blocks):
        qm[i] = block_mean(qf, a, b)
        qc[a:b] = qf[a:b] - qm[i][None]          # float32 subtraction, correctly rounded
    return qc, qm


def quantize(q, k, v, cu_seqlens: List[int], softmax_scale: float = None,
             q_centre: bool = False) -> Dict[str, np.ndarray]:
    """All three tensors.  Keys: q_codes, k_codes, v_codes ([T, H, D] uint8),
    scales ([3, H] float32, rows Q, K, V) and mu ([nseg, H, D] float32).  With
    ``softmax_scale`` given, Q's scale is ``q_scale_pow2`` of its amax/448 scale
    (the product's rule).

    ``q_centre``: Q is replaced by fl32(q - qm) (``centre_q``) before its amax
    and its codes are taken, and the block means come back as ``qm``
    [nq, H, D]; the attention then uses the operand ``qcentre_operand``, the
    dequantized centred Q plus the exact block mean (the mean term qm . k added
    back to the scores without rounding)."""
    rk = quantize_k(k, cu_seqlens)
    qm = None
    if q_centre:
        q, qm = centre_q(q, cu_seqlens)
    rq = quantize_plain(q)
    if softmax_scale is not None:
        rq = quantize_plain(q, q_scale_pow2(rq["scale"], rk["scale"], softmax_scale))
    rv = quantize_plain(v)
    out = {
        "q_codes": rq["codes"], "k_codes": rk["codes"], "v_codes": rv["codes"],
        "scales": np.stack([rq["scale"], rk["scale"], rv["scale"]]).astype(np.float32),
        "mu": rk["mu"],
    }
    if q_centre:
        out["qm"] = qm
    return out


def qcentre_operand(q_codes: np.ndarray, q_scale: np.ndarray, qm: np.ndarray,
                    cu_seqlens: List[int]) -> np.ndarray:
    """float64 Q operand of a Q-centred quantization: e4m3_value(code) * s_q
    plus the block mean of the row's 128-row block (``qm`` in the order of
    ``mxfp4.q_blocks``).  ``q_scale`` is [H], or [nseg, H] for per-segment
    scales."""
    from .mxfp4 import q_blocks
    qs = np.asarray(q_scale, np.float64)
    out = np.zeros(q_codes.shape, np.float64)
    for i, (s, a, b) in enumerate(q_blocks(cu_seqlens)):
        sc = qs[s] if qs.ndim == 2 else qs
        out[a:b] = e4m3.decode(q_codes[a:b]) * sc[None, :, None] + np.asarray(qm[i], np.float64)[None]
    return out


def quantize_segments(q, k, v, cu_seqlens: List[int], softmax_scale: float = None,
                      q_centre: bool = False) -> Dict[str, np.ndarray]:
    """Per-(segment, head) scales: every segment is quantized as if it were the
    whole call, with the per-head rule above applied to that segment's tokens
    only (so no segment's codes depend on another segment's values).

    Keys as ``quantize`` except ``scales`` [3, nseg, H] (rows Q, K, V).  An
    empty segment gets the scales of an all-zero head (1.0, and Q's rounded
    value for it when ``softmax_scale`` is given).  With ``q_centre`` the
    block means of all segments come back as ``qm`` (blocks of
    ``mxfp4.q_blocks``, which never cross a segment boundary).
    """
    qf, kf, vf = _as_f32(q), _as_f32(k), _as_f32(v)
    T, H, D = qf.shape
    nseg = len(cu_seqlens) - 1
    out = {"q_codes": np.zeros((T, H, D), np.uint8), "k_codes": np.zeros((T, H, D), np.uint8),
           "v_codes": np.zeros((T, H, D), np.uint8), "scales": np.zeros((3, nseg, H), np.float32),
           "mu": np.zeros((nseg, H, D), np.float32)}
    qms = []
    for s in range(nseg):
        a, b = cu_seqlens[s], cu_seqlens[s + 1]
        r = quantize(qf[a:b], kf[a:b], vf[a:b], [0, b - a], softmax_scale, q_centre=q_centre)
        for name in ("q_codes", "k_codes", "v_codes"):
            out[name][a:b] = r[name]
        out["scales"][:, s] = r["scales"]
        out["mu"][s] = r["mu"][0]
        if q_centre:
            qms.append(r["qm"])
    if q_centre:
        out["qm"] = np.concatenate(qms, axis=0) if qms else np.zeros((0, H, D), np.float32)
    return out


def dequantize_segments(codes: np.ndarray, scales: np.ndarray, cu_seqlens: List[int]) -> np.ndarray:
    """float64 values of per-(segment, head) codes: scales [nseg, H]."""
    out = np.zeros(codes.shape, np.float64)
    for s in range(len(cu_seqlens) - 1):
        a, b = cu_seqlens[s], cu_seqlens[s + 1]
        out[a:b] = dequantize(codes[a:b], scales[s])
    return out


def dequantize(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """float64 values e4m3_value(code) * s_h (the operands the attention consumes)."""
    return e4m3.decode(codes) * np.asarray(scale, np.float64)[None, :, None]
