"""Pins for the float64 attention oracle (oracle/attention.py).

Each check is independent of the oracle's own code path:
* brute force with mpmath at 50 digits on tiny non-square inputs (catches a
  transposed operand, a dropped scale, a wrong softmax axis or sign);
* closed forms: one dominant key returns exactly its V row (the "one-hot exact"
  check of sglang PR "[DSA] Enable tilelang fp8_e4m3 KV cache on CUDA",
  "Validation"); equal scores return the mean of V; a length-1 segment returns V;
* invariants: segment independence under varlen, per-channel K-shift
  invariance (the reason centring K is exact), permutation equivariance;
* a scrambled-index negative control that must FAIL the comparator (same page,
  "a scrambled-index negative control that must fail").
"""
import math

import mpmath
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import compare


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float64) * scale)


def _mp_attention(q, k, v, cu, sigma):
    mpmath.mp.dps = 50
    T, H, D = q.shape
    out = np.zeros((T, H, D))
    for a, b in zip(cu[:-1], cu[1:]):
        for h in range(H):
            for i in range(a, b):
                sc = [mpmath.mpf(0)] * (b - a)
                for j in range(a, b):
                    acc = mpmath.mpf(0)
                    for d in range(D):
                        acc += mpmath.mpf(float(q[i, h, d])) * mpmath.mpf(float(k[j, h, d]))
                    sc[j - a] = acc * mpmath.mpf(sigma)
                e = [mpmath.exp(s) for s in sc]
                z = mpmath.fsum(e)
                for d in range(D):
                    out[i, h, d] = float(mpmath.fsum(e[j - a] * mpmath.mpf(float(v[j, h, d]))
                                                     for j in range(a, b)) / z)
    return out


@pytest.mark.parametrize("T,H,D,cu", [
    (5, 1, 1, [0, 5]),
    (7, 2, 4, [0, 3, 3, 7]),
    (6, 1, 128, [0, 6]),
    (8, 2, 3, [0, 1, 8]),
])
def test_brute_force_mpmath(T, H, D, cu):
    q = _rand((T, H, D), 1, 0.7)
    k = _rand((T, H, D), 2, 0.9)
    v = _rand((T, H, D), 3)
    scale = 1.0 / math.sqrt(D) if D > 1 else 0.8
    sigma = float(np.float32(scale))
    got = A.attention(q, k, v, cu, scale).numpy()
    exp = _mp_attention(q.numpy(), k.numpy(), v.numpy(), cu, sigma)
    rel = np.abs(got - exp).max() / np.abs(exp).max()
    assert rel <= 1e-13


def test_rows_api_matches_full():
    cu = [0, 40, 40, 97, 100]
    q, k, v = _rand((100, 3, 16), 4), _rand((100, 3, 16), 5), _rand((100, 3, 16), 6)
    full = A.attention(q, k, v, cu, 0.25)
    rows = [0, 5, 39, 40, 41, 96, 97, 99]
    part = A.attention_rows(q, k, v, cu, 0.25, rows)
    # the same definition on fewer rows; BLAS blocking may reorder the float64 sums
    assert torch.allclose(part, full[rows], rtol=0, atol=1e-14)


def test_one_hot_returns_v_row_exactly():
    # key j of every segment has a logit margin >= 60 over all other keys
    T, H, D = 64, 2, 128
    cu = [0, 30, 64]
    q = _rand((T, H, D), 7) * 0.01
    k = _rand((T, H, D), 8) * 0.01
    v = _rand((T, H, D), 9)
    hot = {0: 11, 1: 50}
    for s, j in hot.items():
        a, b = cu[s], cu[s + 1]
        k[j] = 0.0
        k[j, :, 0] = 1.0
        q[a:b, :, 0] = 1000.0    # score_j * sigma = 1000/sqrt(128) ~ 88 >> others
    out = A.attention(q, k, v, cu, 1.0 / math.sqrt(D))
    for s, j in hot.items():
        a, b = cu[s], cu[s + 1]
        assert torch.equal(out[a:b], v[j].unsqueeze(0).expand(b - a, H, D))
        # and the BF16 rounding of that output is the BF16 rounding of v_j
        assert torch.equal(out[a:b].to(torch.bfloat16), v[j].to(torch.bfloat16).expand(b - a, H, D))


def test_equal_scores_give_mean_of_v():
    T, H, D = 50, 2, 128
    cu = [0, 17, 50]
    q = torch.zeros((T, H, D), dtype=torch.float64)
    k, v = _rand((T, H, D), 10), _rand((T, H, D), 11)
    out = A.attention(q, k, v, cu, 0.1)
    for a, b in zip(cu[:-1], cu[1:]):
        mean = v[a:b].mean(dim=0, keepdim=True)
        assert torch.allclose(out[a:b], mean.expand(b - a, H, D), rtol=0, atol=1e-14)


def test_length_one_segment_returns_v():
    T, H, D = 9, 2, 128
    cu = [0, 8, 9]
    q, k, v = _rand((T, H, D), 12), _rand((T, H, D), 13), _rand((T, H, D), 14)
    out = A.attention(q, k, v, cu, 0.088)
    assert torch.equal(out[8], v[8])


def test_segment_independence():
    T, H, D = 120, 2, 32
    cu = [0, 50, 50, 119, 120]
    q, k, v = _rand((T, H, D), 15), _rand((T, H, D), 16), _rand((T, H, D), 17)
    packed = A.attention(q, k, v, cu, 0.17)
    for a, b in zip(cu[:-1], cu[1:]):
        if b <= a:
            continue
        alone = A.attention(q[a:b], k[a:b], v[a:b], [0, b - a], 0.17)
        assert torch.equal(packed[a:b], alone)
    # perturbing another segment changes nothing in this one
    k2, v2 = k.clone(), v.clone()
    k2[60:119] += 5.0
    v2[60:119] *= -3.0
    again = A.attention(q, k2, v2, cu, 0.17)
    assert torch.equal(again[:50], packed[:50]) and torch.equal(again[119:], packed[119:])
    assert not torch.equal(again[50:119], packed[50:119])


def test_k_shift_invariance():
    # a per-(head, channel) constant added to every key of a segment leaves the output unchanged
    T, H, D = 96, 3, 128
    cu = [0, 96]
    q, k, v = _rand((T, H, D), 18), _rand((T, H, D), 19), _rand((T, H, D), 20)
    c = _rand((1, H, D), 21, 2.0)
    o1 = A.attention(q, k, v, cu, 1 / math.sqrt(D))
    o2 = A.attention(q, k + c, v, cu, 1 / math.sqrt(D))
    assert (o1 - o2).abs().max() / o1.abs().max() <= 1e-12


def test_permutation_equivariance():
    T, H, D = 80, 2, 64
    cu = [0, 80]
    q, k, v = _rand((T, H, D), 22), _rand((T, H, D), 23), _rand((T, H, D), 24)
    out = A.attention(q, k, v, cu, 0.125)
    g = torch.Generator().manual_seed(25)
    pq, pk = torch.randperm(T, generator=g), torch.randperm(T, generator=g)
    # permuting queries permutes output rows; permuting key/value rows together changes nothing
    out2 = A.attention(q[pq], k[pk], v[pk], cu, 0.125)
    assert torch.allclose(out2, out[pq], rtol=0, atol=1e-13)


def test_scrambled_index_negative_control_fails():
    """A comparator that cannot tell a wrong answer from a right one is vacuous."""
    T, H, D = 512, 2, 128
    cu = [0, 512]
    g = torch.Generator().manual_seed(26)
    q, k, v = (torch.randn((T, H, D), generator=g, dtype=torch.float64) for _ in range(3))
    ref = A.attention(q, k, v, cu, 1 / math.sqrt(D))
    perm = torch.randperm(T, generator=g)
    scrambled_k = A.attention(q, k[perm], v, cu, 1 / math.sqrt(D))   # K rows shuffled vs V rows
    scrambled_out = ref[perm]                                         # output rows shuffled
    for bad in (scrambled_k, scrambled_out):
        assert not compare.within_bar(bad, ref)
        assert compare.rel_rms(bad, ref) > 0.5
    assert compare.within_bar(ref, ref)


def test_lse_rows_closed_form():
    # equal scores: lse = log(L) + sigma * score
    T, H, D = 33, 2, 8
    q = torch.zeros((T, H, D), dtype=torch.float64)
    k = _rand((T, H, D), 27)
    lse = A.lse_rows(q, k, [0, 33], 0.3, rows=[0, 32])
    assert torch.allclose(lse, torch.full_like(lse, math.log(33)), atol=1e-14)


# ---------------------------------------------------------------- causal variant

def _mp_causal(q, k, v, cu, sigma):
    """mpmath brute force of the causal reading: key j of a segment is visible
    to query i of the same segment when j - a <= i - a."""
    mpmath.mp.dps = 50
    T, H, D = q.shape
    out = np.zeros((T, H, D))
    for a, b in zip(cu[:-1], cu[1:]):
        for h in range(H):
            for i in range(a, b):
                js = list(range(a, i + 1))
                sc = [mpmath.fsum(mpmath.mpf(float(q[i, h, d])) * mpmath.mpf(float(k[j, h, d])) for d in range(D))
                      * mpmath.mpf(sigma) for j in js]
                e = [mpmath.exp(x) for x in sc]
                z = mpmath.fsum(e)
                for d in range(D):
                    out[i, h, d] = float(mpmath.fsum(e[n] * mpmath.mpf(float(v[j, h, d])) for n, j in enumerate(js)) / z)
    return out


@pytest.mark.parametrize("T,H,D,cu", [(6, 1, 3, [0, 6]), (9, 2, 4, [0, 4, 4, 9])])
def test_causal_brute_force_mpmath(T, H, D, cu):
    q, k, v = _rand((T, H, D), 11, 0.8), _rand((T, H, D), 12), _rand((T, H, D), 13)
    got = A.attention(q, k, v, cu, 0.7, causal=True).numpy()
    exp = _mp_causal(q.numpy(), k.numpy(), v.numpy(), cu, float(np.float32(0.7)))
    assert np.abs(got - exp).max() / np.abs(exp).max() <= 1e-13


def test_causal_row_equals_prefix_segment():
    """Row i of a causal segment is the last row of the plain attention over the
    segment's prefix [a, a + i + 1); the first row is its V row."""
    T, H, D = 70, 2, 128
    cu = [0, 33, 70]
    q, k, v = _rand((T, H, D), 21), _rand((T, H, D), 22), _rand((T, H, D), 23)
    got = A.attention(q, k, v, cu, 0.088, causal=True)
    for a, b in zip(cu[:-1], cu[1:]):
        for i in (a, a + 1, (a + b) // 2, b - 1):
            pre = A.attention(q[a:i + 1], k[a:i + 1], v[a:i + 1], [0, i + 1 - a], 0.088)
            torch.testing.assert_close(got[i], pre[-1], rtol=1e-13, atol=1e-13)
        torch.testing.assert_close(got[a], v[a], rtol=1e-14, atol=1e-14)
    # the last row of a segment sees every key: it equals the non-causal row
    full = A.attention(q, k, v, cu, 0.088)
    for b in cu[1:]:
        torch.testing.assert_close(got[b - 1], full[b - 1], rtol=1e-13, atol=1e-13)
    # rows api and LSE agree with the full causal computation
    rows = [0, 5, 32, 33, 50, 69]
    torch.testing.assert_close(A.attention_rows(q, k, v, cu, 0.088, rows, causal=True), got[rows], rtol=1e-13, atol=1e-13)
    lse = A.lse_rows(q, k, cu, 0.088, rows, causal=True)
    for n, r in enumerate(rows):
        a = max(x for x in cu[:-1] if x <= r and r < cu[cu.index(x) + 1])
        sc = (q[r][None] * k[a:r + 1]).sum(-1) * float(np.float32(0.088))      # [keys, H]
        torch.testing.assert_close(lse[n], torch.logsumexp(sc, dim=0), rtol=1e-13, atol=1e-13)


def test_causal_off_by_one_negative_control():
    """A planted mistake (each query also sees the next key) must fail the prefix pin."""
    T, H, D = 40, 1, 16
    q, k, v = _rand((T, H, D), 31), _rand((T, H, D), 32), _rand((T, H, D), 33)
    good = A.attention(q, k, v, [0, T], 0.25, causal=True)
    bad = torch.stack([A.attention(q[:i + 2], k[:i + 2], v[:i + 2], [0, min(i + 2, T)], 0.25)[i] for i in range(T)])
    assert (good - bad).abs().max() > 1e-3


def test_lse_rows_two_keys_closed_form():
    # two keys with exact scores s1, s2 (D = 1): lse = sigma s1 + log(1 + e^(sigma (s2 - s1))),
    # with sigma the float32 value of the scale; a dropped or misapplied sigma, a
    # wrong sign or a wrong key range shows here
    for scale, (x, a, b) in [(0.3, (2.0, 3.0, -5.0)), (0.08838834764831845, (6.0, 7.5, 7.0)),
                             (1.7, (-1.5, 4.0, 2.0))]:
        sigma = float(np.float32(scale))
        q = torch.tensor([[[x]], [[x]]], dtype=torch.float64)
        k = torch.tensor([[[a]], [[b]]], dtype=torch.float64)
        s1, s2 = x * a, x * b
        want = sigma * s1 + math.log1p(math.exp(sigma * (s2 - s1)))
        got = A.lse_rows(q, k, [0, 2], scale, rows=[0, 1]).numpy()
        assert np.allclose(got, want, rtol=0, atol=1e-13)
        # causal: row 0 sees key 0 only, row 1 both
        gc = A.lse_rows(q, k, [0, 2], scale, rows=[0, 1], causal=True).numpy()
        assert abs(gc[0, 0] - sigma * s1) <= 1e-13 and abs(gc[1, 0] - want) <= 1e-13


def test_lse_rows_brute_force_mpmath():
    mpmath.mp.dps = 40
    T, H, D = 6, 2, 3
    q, k = _rand((T, H, D), 61), _rand((T, H, D), 62)
    cu = [0, 2, 6]
    scale = 0.7
    sigma = float(np.float32(scale))
    got = A.lse_rows(q, k, cu, scale).numpy()
    for s, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        for i in range(a, b):
            for h in range(H):
                terms = [mpmath.exp(mpmath.mpf(sigma) * mpmath.fsum(
                    mpmath.mpf(float(q[i, h, d])) * mpmath.mpf(float(k[j, h, d])) for d in range(D)))
                    for j in range(a, b)]
                assert abs(got[i, h] - float(mpmath.log(mpmath.fsum(terms)))) <= 1e-12
