"""Pins for the CPU quantizer (oracle/quantize.py).

* scale: closed form fl32(amax/448) with amax taken by torch, and the all-zero head;
* fixed-order K mean: equals the exactly rounded mean (fractions) where the
  float64 sums are exact, and a hand-worked case where the summation order
  decides the result;
* K amax: the brute-force max |fl32(x - mu)| equals the min/max route
  max(fl32(max - mu), fl32(mu - min)) (rounding is monotone);
* centring: shifting K by a per-channel constant leaves K codes unchanged when
  the mean is exact, and dequantized centred keys give the same attention as
  the raw keys up to quantization error;
* codes of Q and V: one element at a time against the e4m3 brute force in
  tests/test_oracle_e4m3.py is indirect, so here a few elements are checked
  against torch's float8_e4m3fn cast of the same fl32(x/s).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import quantize as Qz
from oracle import e4m3


def _bf16(shape, seed, scale=1.0, offset=0.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale + offset).to(torch.bfloat16)


def test_plain_scale_closed_form_and_codes():
    x = _bf16((300, 3, 128), 1, 2.0)
    x[:, 2] = 0                                     # an all-zero head
    r = Qz.quantize_plain(x)
    amax = x.float().abs().amax(dim=(0, 2)).numpy()
    assert r["scale"][0] == np.float32(amax[0]) / np.float32(448)
    assert r["scale"][1] == np.float32(amax[1]) / np.float32(448)
    assert r["scale"][2] == np.float32(1.0)
    assert np.all(r["codes"][:, 2] == 0)
    # the max element of each head lands exactly on +-448
    for h in range(2):
        flat = x[:, h].float().abs().flatten()
        i = int(flat.argmax())
        assert e4m3.decode(r["codes"][:, h].reshape(-1)[i:i + 1])[0] in (448.0, -448.0)
    ref = (torch.from_numpy(x.float().numpy() / r["scale"][None, :, None])
           .to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    assert np.array_equal(r["codes"], ref)


def test_mean_equals_exact_rational_mean():
    T, H, D = 700, 2, 16
    x = _bf16((T, H, D), 2).float().numpy()
    for a, b in [(0, 700), (0, 256), (13, 600), (699, 700)]:
        mu = Qz.segment_mean(x, a, b)
        for h in range(H):
            for d in range(D):
                exact = sum(Fraction(float(v)) for v in x[a:b, h, d]) / (b - a)
                # bf16 data: float64 partial sums are exact here, so the only
                # roundings are the division and the final float32 cast
                assert mu[h, d] == np.float32(float(exact))


def test_mean_fixed_chunk_order():
    # 257 tokens: chunk 0 = [2^60, 1, 1, ..., 1] (255 ones), chunk 1 = [-2^60].
    # In chunk 0 each +1 is below half an ulp of 2^60 and is lost: chunk sum 2^60.
    # Total = 2^60 + (-2^60) = 0, so mu = 0 (the exact mean would be 255/257).
    x = np.ones((257, 1, 1), np.float32)
    x[0] = 2.0 ** 60
    x[256] = -(2.0 ** 60)
    assert Qz.segment_mean(x, 0, 257)[0, 0] == 0.0
    # with the large values in the same chunk and the ones after, the ones survive
    y = np.ones((257, 1, 1), np.float32)
    y[0] = 2.0 ** 60
    y[1] = -(2.0 ** 60)
    assert Qz.segment_mean(y, 0, 257)[0, 0] == np.float32(255.0 / 257.0)


def test_k_amax_min_max_route_and_mu_layout():
    T, H, D = 600, 2, 128
    cu = [0, 100, 100, 599, 600]
    x = _bf16((T, H, D), 3, 1.0, 0.5)
    r = Qz.quantize_k(x, cu)
    xf = x.float().numpy()
    amax = np.zeros(H, np.float32)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b <= a:
            assert np.all(r["mu"][s] == 0)
            continue
        mx = xf[a:b].max(axis=0)
        mn = xf[a:b].min(axis=0)
        mu = r["mu"][s]
        amax = np.maximum(amax, np.maximum((mx - mu), (mu - mn)).max(axis=1))
    assert np.array_equal(r["scale"], np.float32(amax) / np.float32(448))


def test_k_shift_leaves_codes_unchanged_when_mean_is_exact():
    # K on a 1/16 grid in [-2, 2]; +8 stays exactly representable in bf16 and the
    # segment lengths are powers of two, so mu shifts by exactly 8 and y is unchanged
    g = torch.Generator().manual_seed(4)
    T, H, D = 512, 2, 128
    cu = [0, 256, 512]
    k = (torch.randint(-32, 33, (T, H, D), generator=g).float() / 16).to(torch.bfloat16)
    k8 = (k.float() + 8.0).to(torch.bfloat16)
    assert torch.equal(k8.float() - 8.0, k.float())
    r0, r1 = Qz.quantize_k(k, cu), Qz.quantize_k(k8, cu)
    assert np.array_equal(r0["codes"], r1["codes"])
    assert np.array_equal(r0["scale"], r1["scale"])
    assert np.array_equal(r1["mu"], r0["mu"] + np.float32(8.0))


def test_quantize_bundle_shapes():
    T, H = 130, 2
    q, k, v = _bf16((T, H, 128), 5), _bf16((T, H, 128), 6), _bf16((T, H, 128), 7)
    r = Qz.quantize(q, k, v, [0, 65, 130])
    assert r["q_codes"].shape == (T, H, 128) and r["q_codes"].dtype == np.uint8
    assert r["scales"].shape == (3, H) and r["scales"].dtype == np.float32
    assert r["mu"].shape == (2, H, 128)
    deq = Qz.dequantize(r["v_codes"], r["scales"][2])
    assert np.abs(deq - v.float().numpy()).max() <= float(r["scales"][2].max()) * 16.0


def test_q_scale_pow2_properties():
    # the product's Q scale: at least amax/448, below twice it, and the score
    # factor softmax_scale * s_q * s_k * log2(e) a power of two up to rounding
    rng = np.random.default_rng(11)
    base = np.float32(10.0) ** rng.uniform(-6, 3, 400).astype(np.float32)
    s_k = np.float32(10.0) ** rng.uniform(-6, 3, 400).astype(np.float32)
    for sigma in (1 / np.sqrt(128), 0.05, 1.0, 3.7):
        s = Qz.q_scale_pow2(base, s_k, sigma)
        assert s.dtype == np.float32
        b64, s64 = base.astype(np.float64), s.astype(np.float64)
        assert np.all(s64 >= b64 * (1 - 2.0 ** -22)) and np.all(s64 < 2 * b64)
        c = float(np.float32(sigma)) * s64 * s_k.astype(np.float64) * np.log2(np.e)
        m = np.round(np.log2(c))
        assert np.all(np.abs(c / 2.0 ** m - 1) < 2.0 ** -21)
        # the largest |q| quantizes to a code of magnitude in (224, 448]
        y = (base * np.float32(448)) / s
        assert np.all(y > 224) and np.all(y <= 448 * (1 + 2.0 ** -20))


def test_q_scale_pow2_worked_cases():
    # a factor that is already a power of two keeps the amax/448 scale exactly:
    # softmax_scale * s_k * log2(e) = 2^-3 with s_k = 2^-3 / fl32(sigma * log2e)
    sigma = 1.0 / np.log2(np.e)                 # fl32(sigma) * fl32(log2 e) rounds to 1
    f = np.float32(np.float32(sigma) * np.float32(1.0)) * Qz.LOG2E_F32
    assert f == np.float32(1.0)
    s = Qz.q_scale_pow2(np.float32([0.25, 0.3, 0.5 + 2.0 ** -24]), np.float32([1.0] * 3), sigma)
    assert s[0] == np.float32(0.25)             # t = 2^-2 exactly: m = -2
    assert s[1] == np.float32(0.5)              # t = 0.3: next power of two
    assert s[2] == np.float32(1.0)              # just above 2^-1: m = 0
    # outside the normal float range the plain scale is kept
    tiny = Qz.q_scale_pow2(np.float32([1e-30]), np.float32([1e-20]), 0.1)
    assert tiny[0] == np.float32(1e-30)


def test_quantize_with_softmax_scale_changes_only_q():
    T, H = 200, 2
    q, k, v = _bf16((T, H, 128), 21), _bf16((T, H, 128), 22, 1.5), _bf16((T, H, 128), 23)
    cu = [0, 77, 200]
    r0 = Qz.quantize(q, k, v, cu)
    r1 = Qz.quantize(q, k, v, cu, 1 / np.sqrt(128))
    for key in ("k_codes", "v_codes", "mu"):
        assert np.array_equal(r0[key], r1[key])
    assert np.array_equal(r0["scales"][1:], r1["scales"][1:])
    assert np.array_equal(r1["scales"][0], Qz.q_scale_pow2(r0["scales"][0], r0["scales"][1], 1 / np.sqrt(128)))
    # Q codes against torch's E4M3 cast of fl32(q / s) at the new scale
    ref = (torch.from_numpy(q.float().numpy() / r1["scales"][0][None, :, None])
           .to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    assert np.array_equal(r1["q_codes"], ref)


def test_segment_scales_single_segment_is_per_head():
    q, k, v = _bf16((300, 3, 128), 11), _bf16((300, 3, 128), 12, 1.0, 0.7), _bf16((300, 3, 128), 13)
    a = Qz.quantize(q, k, v, [0, 300], 0.088)
    b = Qz.quantize_segments(q, k, v, [0, 300], 0.088)
    for name in ("q_codes", "k_codes", "v_codes", "mu"):
        assert np.array_equal(a[name], b[name]), name
    assert np.array_equal(a["scales"], b["scales"][:, 0])


def test_segment_scales_are_independent_of_other_segments():
    cu = [0, 130, 130, 400, 401]
    q, k, v = _bf16((401, 2, 128), 21), _bf16((401, 2, 128), 22), _bf16((401, 2, 128), 23)
    base = Qz.quantize_segments(q, k, v, cu, 0.088)
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    q2[130:400] *= 7
    k2[130:400] += 3
    v2[130:400] *= 0.01
    pert = Qz.quantize_segments(q2, k2, v2, cu, 0.088)
    for name in ("q_codes", "k_codes", "v_codes"):
        assert np.array_equal(base[name][:130], pert[name][:130]), name
        assert np.array_equal(base[name][400:], pert[name][400:]), name
    for s in (0, 1, 3):
        assert np.array_equal(base["scales"][:, s], pert["scales"][:, s])
    # the empty segment carries the all-zero-head scales
    assert np.all(base["scales"][1, 1] == 1.0) and np.all(base["scales"][2, 1] == 1.0)
    # per-head scales over the whole call would have changed segment 0's V codes
    ph = Qz.quantize(q, k, v2, cu, 0.088)["v_codes"][:130]
    assert not np.array_equal(ph, Qz.quantize(q, k, v, cu, 0.088)["v_codes"][:130])


def test_segment_scales_power_of_two_rescaling():
    cu = [0, 200, 333]
    q, k, v = _bf16((333, 2, 128), 31), _bf16((333, 2, 128), 32), _bf16((333, 2, 128), 33)
    base = Qz.quantize_segments(q, k, v, cu)
    v2 = v.clone()
    v2[200:] *= 8                                     # exact in bf16
    r = Qz.quantize_segments(q, k, v2, cu)
    assert np.array_equal(r["v_codes"], base["v_codes"])
    assert np.array_equal(r["scales"][2, 1], base["scales"][2, 1] * np.float32(8))
    assert np.array_equal(r["scales"][2, 0], base["scales"][2, 0])
    # dequantized values follow the scaling exactly
    dv = Qz.dequantize_segments(r["v_codes"], r["scales"][2], cu)
    db = Qz.dequantize_segments(base["v_codes"], base["scales"][2], cu)
    assert np.array_equal(dv[200:], 8 * db[200:]) and np.array_equal(dv[:200], db[:200])


# ------------------------------------------------------------------------------
# Q's power-of-two scale, bit for bit, from exact rational arithmetic.  Every
# float32 operation of the rule (products, the quotient) is evaluated exactly
# with fractions.Fraction and rounded to float32 by the format's definition
# (nearest, ties to even, subnormal quantum 2^-149); the power of two is the
# smallest 2^m >= t found by search over m, not by frexp.


def _fl32(x: Fraction) -> Fraction:
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = math.floor(math.log2(float(a)))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    n = a / quantum
    whole = n.numerator // n.denominator
    rem = n - whole
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and whole % 2 == 1):
        whole += 1
    return sign * whole * quantum


def _q_scale_exact(amax_q: float, amax_k: float, sigma: float) -> np.float32:
    base = _fl32(Fraction(amax_q) / 448) if amax_q > 0 else Fraction(1)
    s_k = _fl32(Fraction(amax_k) / 448) if amax_k > 0 else Fraction(1)
    sig = _fl32(Fraction(sigma))                              # the float32 kernel argument
    log2e = _fl32(Fraction(1.4426950408889634))
    f = _fl32(_fl32(sig * s_k) * log2e)
    t = _fl32(f * base)
    if not (Fraction(2) ** -126 <= t < Fraction(2) ** 126):
        return np.float32(float(base))
    m = next(m for m in range(-160, 160) if Fraction(2) ** m >= t)
    return np.float32(float(_fl32(Fraction(2) ** m / f)))


def _bf16_values(n, seed, lo, hi):
    rng = np.random.default_rng(seed)
    x = (10.0 ** rng.uniform(lo, hi, n)).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy()   # amax of BF16 data is a BF16 value


@pytest.mark.parametrize("sigma", [1 / math.sqrt(128), 1 / math.sqrt(64), 0.05, 0.3, 1.0, 3.7])
def test_q_scale_pow2_bits_match_exact_arithmetic(sigma):
    aq, ak = _bf16_values(300, 31, -3, 3), _bf16_values(300, 32, -3, 3)
    base = Qz.head_scale(aq)
    s_k = Qz.head_scale(ak)
    got = Qz.q_scale_pow2(base, s_k, sigma)
    want = np.array([_q_scale_exact(float(a), float(b), sigma) for a, b in zip(aq, ak)], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_q_scale_pow2_bits_where_t_is_a_power_of_two():
    # cases where fl32(f * base) lands exactly on 2^k: m must be k itself (an
    # off-by-one in the smallest power of two shows here and nowhere else)
    rng = np.random.default_rng(33)
    sigma = 0.08838834764831845
    hits = 0
    for _ in range(4000):
        ak = float(_bf16_values(1, int(rng.integers(1 << 30)), -2, 2)[0])
        s_k = Qz.head_scale(np.float32([ak]))
        f = (np.float32(sigma) * s_k) * Qz.LOG2E_F32
        k = int(rng.integers(-8, 4))
        base = (np.float32(2.0 ** k) / f).astype(np.float32)
        if (f * base).astype(np.float32)[0] != np.float32(2.0 ** k):
            continue
        aq = base.astype(np.float64)[0] * 448.0
        if np.float32(aq) / np.float32(448) != base[0]:
            continue
        hits += 1
        got = Qz.q_scale_pow2(base, s_k, sigma)[0]
        assert got == _q_scale_exact(aq, ak, sigma) == base[0]
    assert hits >= 20
