"""The error range of the default (log-linear) E4M3 probability code, which
bounds the LSE of default plans against the exact log-sum-exp (CPU only).

Code c = rne(y) for y = 8 x + LOGLIN_BIAS; the weight is the E4M3 value of c;
the exact probability in the same frame is 2^((y - LOGLIN_BIAS) / 8).  On the
half-open interval of y that rounds to c the exact value is monotone, so the
ratio's extremes over all y are at the interval ends of the normal codes.
"""
import numpy as np

from oracle import e4m3
from tests.cases import LOGLIN_BIAS, LOGLIN_RATIO_MAX, LOGLIN_RATIO_MIN


def _ratio_extremes():
    c = np.arange(8, 127)
    v = e4m3.decode(c.astype(np.uint8)).astype(np.float64)
    lo = v / 2.0 ** ((c + 0.5 - LOGLIN_BIAS) / 8)      # y at the top of c's interval
    hi = v / 2.0 ** ((c - 0.5 - LOGLIN_BIAS) / 8)      # y at the bottom
    return lo.min(), hi.max()


def test_ratio_range_is_the_stated_one():
    lo, hi = _ratio_extremes()
    assert LOGLIN_RATIO_MIN <= lo < LOGLIN_RATIO_MIN + 1e-4
    assert LOGLIN_RATIO_MAX - 1e-4 < hi <= LOGLIN_RATIO_MAX


def test_ratio_range_by_sampling():
    # the same range from dense samples of y (no interval reasoning)
    y = np.linspace(7.5001, 126.4999, 1_000_003)
    c = np.rint(y).astype(np.int64)
    v = e4m3.decode(c.astype(np.uint8)).astype(np.float64)
    r = v / 2.0 ** ((y - LOGLIN_BIAS) / 8)
    assert LOGLIN_RATIO_MIN <= r.min() and r.max() <= LOGLIN_RATIO_MAX
    assert r.min() < LOGLIN_RATIO_MIN + 1e-4 and r.max() > LOGLIN_RATIO_MAX - 1e-4


def test_reference_code_is_112():
    # the kernel puts its reference maximum on y = 110, the code of 112
    assert float(e4m3.decode(np.array([110], np.uint8))[0]) == 112.0
    assert abs(2.0 ** ((110 - LOGLIN_BIAS) / 8) - 112.0) < 1e-6
