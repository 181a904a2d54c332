"""Shared helpers of the GPU parity tests (test infrastructure)."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import fp8_flash_attention_amd as fa
from fp8_flash_attention_amd import _lib


def log(msg: str) -> None:
    """Name the case before GPU work so a fault can be attributed."""
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def v_key_position(kk: np.ndarray) -> np.ndarray:
    """Position inside its 64-key group at which the workspace V layout stores key kk (0..63).

    Documented layout: byte p = 32*j + 16*b + 4*r + i holds key 32*b + 8*r + 4*j + i.
    """
    b = kk // 32
    r = (kk % 32) // 8
    j = (kk % 8) // 4
    i = kk % 4
    return 32 * j + 16 * b + 4 * r + i


def read_codes(plan: fa.Plan, ws: torch.Tensor, heads=None):
    """Workspace codes in canonical [T][H'][128] order (H' = the requested heads), plus
    scales [3][H], mu [nseg][H][128], and the padding bytes of every region."""
    cu = plan.cu_seqlens
    T = plan.tokens
    Hs = list(range(plan.heads)) if heads is None else list(heads)
    qr = plan.region(ws, _lib.REGION_Q)[Hs].cpu().numpy()      # [H', rows, 128]
    kr = plan.region(ws, _lib.REGION_K)[Hs].cpu().numpy()
    vr = plan.region(ws, _lib.REGION_V)[Hs].cpu().numpy()      # [H', 128, rows]
    scales = plan.region(ws, _lib.REGION_SCALES).cpu().numpy()
    mu = plan.region(ws, _lib.REGION_MU).cpu().numpy()
    rows = qr.shape[1]
    row_of_token = np.zeros(T, np.int64)
    vpos_of_token = np.zeros(T, np.int64)
    used = np.zeros(rows, bool)
    r0 = 0
    for a, b in zip(cu[:-1], cu[1:]):
        L = b - a
        rel = np.arange(L)
        row_of_token[a:b] = r0 + rel
        vpos_of_token[a:b] = r0 + 64 * (rel // 64) + v_key_position(rel % 64)
        used[r0 + rel] = True
        r0 += (L + 127) // 128 * 128
    q = qr[:, row_of_token, :].transpose(1, 0, 2)
    k = kr[:, row_of_token, :].transpose(1, 0, 2)
    v = vr[:, :, vpos_of_token].transpose(2, 0, 1)
    # V padding positions: every position not holding a token
    vused = np.zeros(rows, bool)
    vused[vpos_of_token] = True
    pads = {"q": qr[:, ~used, :], "k": kr[:, ~used, :], "v": vr[:, :, ~vused]}
    return {"q_codes": np.ascontiguousarray(q), "k_codes": np.ascontiguousarray(k),
            "v_codes": np.ascontiguousarray(v), "scales": scales, "mu": mu, "pads": pads}


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 7)


def check_lse(got: np.ndarray, ref_deq: np.ndarray, exact_probs: bool, what: str = "") -> None:
    """LSE of an E4M3 plan against the exact log-sum-exp of the dequantized
    operands' uncentred scores.  The kernel's LSE is the log of the weights
    applied to V (the row's normalizer), each 2^x times a factor in [lo, hi]:
    with exact probabilities E4M3's round-to-nearest bound [1 - 2^-4, 1 + 2^-4]
    on its normal codes, with the default log-linear code [LOGLIN_RATIO_MIN,
    LOGLIN_RATIO_MAX] (tests/cases.py).  So every row lies in that log range
    (plus 2e-3 of FP32 slack) and, as both codes' errors are centred, the
    median row error is small."""
    from tests.cases import LOGLIN_RATIO_MAX, LOGLIN_RATIO_MIN
    lo, hi = (1 - 2.0 ** -4, 1 + 2.0 ** -4) if exact_probs else (LOGLIN_RATIO_MIN, LOGLIN_RATIO_MAX)
    d = np.asarray(got, np.float64) - np.asarray(ref_deq, np.float64)
    assert np.isfinite(d).all()
    med = float(np.median(d))
    log(f"  {what} lse err vs dequantized: min {d.min():.5f} max {d.max():.5f} median {med:.5f}")
    assert d.min() >= np.log(lo) - 2e-3 and d.max() <= np.log(hi) + 2e-3
    assert abs(med) <= 0.01
