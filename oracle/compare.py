"""Comparators for the attention output.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* relative RMS error ``||o - r||_2 / ||r||_2`` over every element, in float64.
  The pages quote a "relative RMS" for E4M3 Q/K/V against a BF16 reference
  without defining it (sglang PR "[diffusion] attention: add fp8_fa_sm120
  FP8 backend for SM120 GPUs", "Accuracy Tests"); this is the plain reading.
* max absolute error, compared with the FP8 operator tolerance 0.1 named on
  the FlashInfer "minimax_h3_sm120_varlen_attention_nvfp4" page (read as an
  element-wise absolute bound, rtol 0).
"""
from __future__ import annotations

import numpy as np
import torch

REL_RMS_BAR = 0.06
ATOL_BAR = 0.1


def _f64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def rel_rms(o, r) -> float:
    o, r = _f64(o), _f64(r)
    den = float(np.sqrt(np.sum(r * r)))
    num = float(np.sqrt(np.sum((o - r) ** 2)))
    return num / den if den > 0 else num


def max_abs(o, r) -> float:
    o, r = _f64(o), _f64(r)
    return float(np.max(np.abs(o - r))) if o.size else 0.0


def within_bar(o, r) -> bool:
    return rel_rms(o, r) <= REL_RMS_BAR and max_abs(o, r) <= ATOL_BAR
