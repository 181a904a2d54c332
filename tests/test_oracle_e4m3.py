"""Pins for the CPU E4M3 encoder (oracle/e4m3.py).

The encoder is checked against things other than itself:
* an exhaustive brute-force nearest-value search over every BF16 bit pattern,
  written here from the format definition (its own value table, its own
  tie-break), at several scales;
* PyTorch's ``float8_e4m3fn`` cast, a library implementation of the same format;
* the worked values in ``tests/golden/e4m3_worked_values.txt`` (OCP OFP8
  specification, Table 1, plus round-to-nearest-even tie cases).
"""
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_worked_values.txt")


def _value_table():
    """Magnitude of every non-negative finite E4M3 code 0x00..0x7E, from the format definition."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(m / 8.0 * 2.0 ** (1 - 7))          # subnormal: 0.m * 2^(1-bias)
        else:
            vals.append((1.0 + m / 8.0) * 2.0 ** (e - 7))  # normal: 1.m * 2^(e-bias)
    return np.array(vals, dtype=np.float64)


def _brute_force(y: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3 magnitude by search; ties go to the even code; sign copied."""
    tab = _value_table()
    # every magnitude >= 1024 has the same nearest finite value as 1024 (the largest, 448);
    # clamping keeps the float64 distances below exact so the search cannot see false ties
    a = np.minimum(np.abs(y.astype(np.float64)), 1024.0)
    d = np.abs(a[:, None] - tab[None, :])                   # [N, 127]
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates prefer an even code (mantissa LSB 0); a tie always pairs
    # two neighbouring codes, exactly one of which is even
    even = (np.arange(0x7F) % 2 == 0)[None, :]
    pick_even = cand & even
    has_even = pick_even.any(axis=1)
    idx = np.where(has_even, pick_even.argmax(axis=1), cand.argmax(axis=1))
    sign = np.signbit(y).astype(np.int64) << 7
    return (idx | sign).astype(np.uint8)


def _all_bf16_as_f32():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    f = bits.view(np.float32)
    return f[np.isfinite(f)]


@pytest.mark.parametrize("scale", [1.0, 1.0 / 448.0 * 3.0, 2.0 ** -7, 0.7071067690849304])
def test_exhaustive_bf16_against_brute_force(scale):
    x = _all_bf16_as_f32()
    with np.errstate(over="ignore"):
        y = (x / np.float32(scale)).astype(np.float32)
    y = y[np.isfinite(y)]
    got = e4m3.encode(y)
    exp = _brute_force(y)
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first y={y[bad[0]]!r} got={got[bad[0]]:#x} exp={exp[bad[0]]:#x}"


def test_dense_float32_grid_against_brute_force():
    # every float32 with a 12-bit mantissa grid between 2^-12 and 2^9, both signs:
    # exercises all tie points of the 3-bit mantissa and the subnormal ties
    e = np.arange(-12, 10)
    m = np.arange(0, 1 << 12) / float(1 << 12)
    y = ((1.0 + m)[None, :] * np.exp2(e)[:, None]).ravel().astype(np.float32)
    y = np.concatenate([y, -y])
    assert np.array_equal(e4m3.encode(y), _brute_force(y))


def test_matches_torch_float8_e4m3fn_cast():
    x = _all_bf16_as_f32()
    x = x[np.abs(x) < 464.0]
    got = e4m3.encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_golden_worked_values():
    n = 0
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            val, code = line.split()[:2]
            y = np.float32(float(val))
            assert int(e4m3.encode(np.array([y]))[0]) == int(code, 16), line
            n += 1
    assert n >= 15


def test_nan_and_inf():
    got = e4m3.encode(np.array([np.nan, -np.nan, np.inf, -np.inf], np.float32))
    assert got[0] & 0x7F == 0x7F and got[2] == 0x7E and got[3] == 0xFE


def test_decode_roundtrip_every_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3.decode(codes)
    finite = ~np.isnan(vals)
    assert finite.sum() == 254                 # only S.1111.111 is NaN
    assert np.array_equal(e4m3.encode(vals[finite].astype(np.float32)), codes[finite])
    assert np.nanmax(vals) == 448.0 and np.nanmin(vals) == -448.0
