"""CPU E4M3 encoder and decoder (OCP 8-bit floating point, E4M3 "FN" variant).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product path
never does.

Format (OCP "8-bit Floating Point Specification (OFP8)", E4M3 encoding):
sign bit, 4 exponent bits with bias 7, 3 mantissa bits.  Exponent field 0
holds subnormals ``m * 2**-9``; exponent fields 1..15 hold ``(1 + m/8) *
2**(e - 7)``; the single pattern S.1111.111 is NaN and there are no
infinities, so the largest finite magnitude is 448 (code 0x7E).

Encoding reading (the pages name E4M3 for Q, K, V and P but fix no rounding
rule; sglang PR "[diffusion] attention: add fp8_fa_sm120 FP8 backend for
SM120 GPUs", "Modifications"): round to nearest, ties to the even mantissa,
subnormals kept, sign copied (so -0.0 encodes as 0x80), magnitudes that round
above 448 saturate to 448, NaN encodes as 0x7F with the sign bit copied.

Parity pins live in ``tests/test_oracle_e4m3.py``.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6


def encode(y) -> np.ndarray:
    """Encode float32 values as E4M3 codes (uint8), element by element.

    Every step is exact in float64 because the input is float32: ``frexp``
    splits off the exponent exactly, scaling by powers of two is exact, and
    ``np.round`` rounds half to even.
    """
    y = np.asarray(y, dtype=np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        return _encode(y)


def _encode(y: np.ndarray) -> np.ndarray:
    a = np.abs(y.astype(np.float64))
    sign = np.signbit(y).astype(np.int64) << 7

    # Normal range: a = f * 2**e with f in [1, 2).
    f2, e2 = np.frexp(a)                 # a = f2 * 2**e2, f2 in [0.5, 1)
    e = e2.astype(np.int64) - 1
    frac8 = (2.0 * f2 - 1.0) * 8.0       # mantissa in units of 1/8, exact
    normal = (e + 7) * 8 + np.round(frac8).astype(np.int64)   # carry into exponent is automatic

    # Subnormal range: a < 2**-6, encoded as round(a / 2**-9); 8 is the smallest normal.
    sub = np.round(a * 2.0 ** 9).astype(np.int64)

    mag = np.where(a < _MIN_NORMAL, sub, normal)
    mag = np.where(np.isfinite(a) & (mag <= 0x7E), mag, 0x7E)   # saturate (incl. +-inf)
    mag = np.where(np.isnan(a), 0x7F, mag)
    return (mag | sign).astype(np.uint8)


def decode(code) -> np.ndarray:
    """Value (float64) of each E4M3 code; NaN for S.1111.111."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return s * val
