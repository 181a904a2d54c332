"""CPU float64 reference for segment-wise dense non-causal attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the product path.

Definition followed (FlashInfer "minimax_h3_sm120_varlen_attention_nvfp4"
page, the formula for ``out[a:b, h]`` and the ``cu_seqlens`` parameter): for
every segment ``[a, b)`` of ``cu_seqlens`` and every head ``h``

    out[a:b, h] = softmax(q[a:b, h] @ k[a:b, h]^T * softmax_scale) @ v[a:b, h]

The softmax runs along the key axis.  The segments partition ``[0, T)``
(``cu_seqlens`` starts at 0, never decreases and ends at T), so every row of
the output is defined; an empty segment has no rows.  Inputs are widened
exactly to float64 and the scale is taken as ``float64(float32(scale))``, the
value a float32 kernel argument carries.  The maximum is subtracted before the
exponential only to keep exp() in range; softmax is unchanged by it.

Causal variant (``causal=True``; the pages send causal attention to another
backend and do not define it, so this is the plain reading for
self-attention): query i of a segment attends to the keys j <= i of the same
segment, positions counted from the segment start.

FP8 recipe (``attention_fp8_recipe``): the arithmetic of the FP8 method of
sglang PR "[diffusion] attention: add fp8_fa_sm120 FP8 backend for SM120
GPUs" ("Modifications": E4M3 operands for both products, an FP32 softmax, the
probabilities packed to E4M3 before the second product), written out per row
without blocking: scores from the dequantized E4M3 operands, the row maximum
mapped to 448 (the top of E4M3; the page does not say where the maximum lands,
and this is the plainest reading that uses the format's whole range), each
probability rounded to float32 and then to E4M3, and the output normalized by
the sum of those E4M3 weights (the weights that actually multiply V).  It shows
how far the method itself, with no blocking, reordering or kernel choices, is
from the exact result; the pins are in the same test file (equal scores,
one dominant key, inputs whose probabilities are powers of two so every
rounding is exact, and a planted missing scale).

Parity pins live in ``tests/test_oracle_attention.py``.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import numpy as np
import torch

ROW_BLOCK = 1024


def _f64(x) -> torch.Tensor:
    if isinstance(x, np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    return x.detach().to("cpu").to(torch.float64)


def _sigma(softmax_scale: float) -> float:
    return float(np.float32(softmax_scale))


def _causal_mask(qpos, L: int) -> torch.Tensor:
    """[R, L] True where key j lies after query position qpos[r] (segment-relative)."""
    return torch.arange(L)[None, :] > torch.as_tensor(qpos, dtype=torch.long)[:, None]


def _segment_rows(qs: torch.Tensor, ks: torch.Tensor, vs: torch.Tensor, sigma: float,
                  qpos=None) -> torch.Tensor:
    """softmax(qs ks^T sigma) vs for one segment; qs [R, H, D], ks/vs [L, H, D].
    With ``qpos`` (segment-relative positions of the R query rows) keys after
    each query are excluded (causal)."""
    qh = qs.permute(1, 0, 2)                       # [H, R, D]
    kh = ks.permute(1, 2, 0)                       # [H, D, L]
    vh = vs.permute(1, 0, 2)                       # [H, L, D]
    s = torch.matmul(qh, kh) * sigma               # [H, R, L]
    if qpos is not None:
        s = s.masked_fill(_causal_mask(qpos, ks.shape[0])[None], -math.inf)
    m = s.max(dim=-1, keepdim=True).values
    p = torch.exp(s - m)
    l = p.sum(dim=-1, keepdim=True)
    o = torch.matmul(p, vh) / l                    # [H, R, D]
    return o.permute(1, 0, 2)                      # [R, H, D]


def attention(q, k, v, cu_seqlens: Sequence[int], softmax_scale: float, causal: bool = False) -> torch.Tensor:
    """Full output, float64 [T, H, D]."""
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    T, H, D = qd.shape
    out = torch.zeros((T, H, D), dtype=torch.float64)
    sigma = _sigma(softmax_scale)
    for a, b in zip(cu_seqlens[:-1], cu_seqlens[1:]):
        if b <= a:
            continue
        for r0 in range(a, b, ROW_BLOCK):
            r1 = min(r0 + ROW_BLOCK, b)
            qpos = list(range(r0 - a, r1 - a)) if causal else None
            out[r0:r1] = _segment_rows(qd[r0:r1], kd[a:b], vd[a:b], sigma, qpos)
    return out


def attention_rows(q, k, v, cu_seqlens: Sequence[int], softmax_scale: float,
                   rows: List[int], causal: bool = False) -> torch.Tensor:
    """Output rows ``rows`` only (each against its own segment), float64 [len(rows), H, D].

    Every query row of the definition is independent of the others, so this is
    the same definition evaluated on a subset of rows.
    """
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    sigma = _sigma(softmax_scale)
    cu = list(cu_seqlens)
    out = torch.zeros((len(rows), qd.shape[1], qd.shape[2]), dtype=torch.float64)
    # group the requested rows by segment
    seg_of = np.searchsorted(np.asarray(cu), np.asarray(rows, dtype=np.int64), side="right") - 1
    for s in sorted(set(seg_of.tolist())):
        a, b = cu[s], cu[s + 1]
        idx = [i for i, ss in enumerate(seg_of.tolist()) if ss == s]
        sel = torch.tensor([rows[i] for i in idx], dtype=torch.long)
        for c0 in range(0, len(idx), ROW_BLOCK):
            part = sel[c0:c0 + ROW_BLOCK]
            qpos = (part - a).tolist() if causal else None
            out[torch.tensor(idx[c0:c0 + ROW_BLOCK])] = _segment_rows(qd[part], kd[a:b], vd[a:b], sigma, qpos)
    return out


def lse_rows(q, k, cu_seqlens: Sequence[int], softmax_scale: float,
             rows: Optional[List[int]] = None, causal: bool = False) -> torch.Tensor:
    """Natural-log log-sum-exp of the scaled scores per (row, head), float64 [R, H]."""
    qd, kd = _f64(q), _f64(k)
    sigma = _sigma(softmax_scale)
    cu = list(cu_seqlens)
    if rows is None:
        rows = list(range(qd.shape[0]))
    out = torch.zeros((len(rows), qd.shape[1]), dtype=torch.float64)
    for i, r in enumerate(rows):
        s = int(np.searchsorted(np.asarray(cu), r, side="right") - 1)
        a, b = cu[s], cu[s + 1]
        kend = r + 1 if causal else b               # causal: keys up to the query itself
        sc = torch.einsum("hd,lhd->hl", qd[r], kd[a:kend]) * sigma
        out[i] = torch.logsumexp(sc, dim=-1)
    return out


FP8_P_TOP = 448.0   # where the row maximum of the probabilities lands (the largest E4M3 value)


def attention_fp8_recipe(q, k, v, cu_seqlens: Sequence[int], softmax_scale: float, causal: bool = False,
                         rows: Optional[List[int]] = None) -> torch.Tensor:
    """The FP8 recipe per row (see the module text), float64 [T or len(rows), H, D].

    ``q``, ``k``, ``v`` are the dequantized E4M3 operands (code value times scale);
    K may be the centred one, since a per-segment constant added to every key
    moves every score of a query and its maximum by the same amount.
    """
    from . import e4m3
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    T, H, D = qd.shape
    sigma = _sigma(softmax_scale)
    cu = list(cu_seqlens)
    if rows is None:
        rows = list(range(T))
    out = torch.zeros((len(rows), H, D), dtype=torch.float64)
    seg_of = np.searchsorted(np.asarray(cu), np.asarray(rows, dtype=np.int64), side="right") - 1
    for i, r in enumerate(rows):
        s_ = int(seg_of[i])
        a, b = cu[s_], cu[s_ + 1]
        kend = r + 1 if causal else b
        sc = torch.einsum("hd,lhd->hl", qd[r], kd[a:kend]) * sigma            # [H, keys]
        m = sc.max(dim=-1, keepdim=True).values
        p32 = (torch.exp(sc - m) * FP8_P_TOP).numpy().astype(np.float32)      # FP32 probabilities
        ph = torch.from_numpy(e4m3.decode(e4m3.encode(p32)))                   # their E4M3 values
        out[i] = torch.einsum("hl,lhd->hd", ph, vd[a:kend]) / ph.sum(dim=-1, keepdim=True)
    return out
