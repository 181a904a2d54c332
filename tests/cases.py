"""Small seeded workloads shared by GPU parity tests and the CPU tests of the
oracle that justify their bars (inputs only: segment tables and seeds)."""
import numpy as np

from workloads import make_workload


def random_varlen():
    """Thirty segments with lengths around the tile edges (0, 1, 63, 64, 65, 127 ...)."""
    rng = np.random.default_rng(101)
    edges = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300, 511, 513]
    lens = list(rng.choice(edges, size=30))
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + int(L))
    return make_workload("rand_varlen", cu[-1], 3, cu, seed=101)


CAUSAL_CASES = [
    make_workload("c256", 256, 2, [0, 256], seed=401),
    make_workload("c_ragged", 700, 4, [0, 300, 700], seed=402, k_offset_var=2.0),
    make_workload("c_varlen", 1500, 3, [0, 0, 1, 64, 65, 193, 700, 700, 1500], seed=403),
    make_workload("c_long", 1200, 2, [0, 1200], seed=404, k_offset_var=2.0),
]

# rows that see fewer keys than this are held to the element-wise bar against
# the dequantized-operand oracle instead of the exact inputs (see
# tests/test_oracle_fp8_recipe.py for why, and why this many)
FEW_KEYS = 64


def visible_keys(cu_seqlens, causal):
    """Keys each row attends to: its segment's length, or (causal) its position + 1."""
    cu = list(cu_seqlens)
    out = np.zeros(cu[-1], np.int64)
    for a, b in zip(cu[:-1], cu[1:]):
        out[a:b] = np.arange(1, b - a + 1) if causal else b - a
    return out


# The default E4M3 probability of a score is the E4M3 value of the code
# rne(y), y = 8 x + LOGLIN_BIAS with x in log2 units (the reference frame
# shifts y by whole multiples of 8, which scales normal E4M3 values by exact
# powers of two).  On E4M3's normal codes (8 .. 126) the weight is 2^x times
# a factor in [LOGLIN_RATIO_MIN, LOGLIN_RATIO_MAX] (tests/test_loglinear_bounds.py
# derives the range), so the log of a row's weight sum (the LSE of default
# plans) lies within [ln MIN, ln MAX] of the exact log-sum-exp of the same
# scores.
LOGLIN_BIAS = 55.54116061995
LOGLIN_RATIO_MIN = 0.9202
LOGLIN_RATIO_MAX = 1.0645
