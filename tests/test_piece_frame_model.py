"""A CPU model of the per-row frame arithmetic of the attention kernel's key
pieces, showing why keys past the end of a range must be masked.

The kernel keeps, per query row, a reference offset nb so that x = c*s + nb
(c the score factor in log2 units); the first tile sets the reference from its
maximum (mapped to log2 112), a later tile moves it only when its largest x
would exceed log2 448 (the largest E4M3 value), and O and l are rescaled by
2^shift when it moves.  p = E4M3(2^x); l sums the E4M3 weights of the real
keys and O the weighted V rows; a piece reports O/l and its log2 weight
w = log2 l - nb, and the combine merges pieces by 2^(w_i - max w).

Keys past the end of a ragged last tile have zero codes, so their score is
exactly 0.  Over a whole segment that is harmless (centred keys average to
zero, so some real score is >= 0), but one piece of a split item can hold only
keys whose scores are all far below 0: an unmasked padded key then moves the
reference to itself, the real weights flush to zero and the piece's output
becomes 0/0.  The model below reproduces that failure and shows that masking
the padded keys (score -inf) removes it; the GPU regression test runs the
same situation through the library.

This is a model of the kernel's frame rules written from their description,
for the argument only: it shares no code with the HIP path and is not the
oracle (the expected values here are the plain float64 softmax).
"""
import numpy as np

from oracle import e4m3

LOG2_REF = np.float32(np.log2(112.0))
LOG2_MAX = np.float32(np.log2(448.0))
TILE = 64


def _e4m3_values(x: np.ndarray) -> np.ndarray:
    return e4m3.decode(e4m3.encode(x.astype(np.float32))).astype(np.float32)


def piece_frame(x: np.ndarray, v: np.ndarray, n_real: int, mask_pad: bool):
    """One query row over a key range of whole tiles: x [keys] scores in log2
    units (padded keys past n_real hold 0, as zero codes score), v [keys, D]
    (padded rows 0).  Returns (O / l, w) in float32 as the kernel computes them."""
    x = x.astype(np.float32).copy()
    if mask_pad:
        x[n_real:] = -np.inf
    nkeys, D = v.shape
    O = np.zeros(D, np.float32)
    l = np.float32(0.0)
    nb = np.float32(0.0)
    for t in range(0, nkeys, TILE):
        xt = x[t:t + TILE]
        if t == 0:
            nb = LOG2_REF - xt.max()
        elif xt.max() + nb > LOG2_MAX:
            shift = LOG2_REF - (xt.max() + nb)
            nb = np.float32(nb + shift)
            a = np.float32(2.0) ** shift
            O, l = (O * a).astype(np.float32), np.float32(l * a)
        p = _e4m3_values(np.exp2((xt + nb).astype(np.float32)))
        real = np.arange(t, t + len(xt)) < n_real
        l = np.float32(l + p[real].sum(dtype=np.float32))
        O = (O + (p[:, None] * v[t:t + TILE]).sum(axis=0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = (O / l).astype(np.float32)
        w = np.float32(np.log2(l) - nb)
    return out, w


def combine(pieces):
    w = np.array([p[1] for p in pieces], np.float64)
    m = w.max()
    a = np.exp2(w - m)
    return sum(ai * p[0].astype(np.float64) for ai, p in zip(a, pieces)) / a.sum()


def _exact(x, v, n_real):
    xs = x[:n_real].astype(np.float64)
    p = np.exp2(xs - xs.max())
    return (p[:, None] * v[:n_real]).sum(axis=0) / p.sum(), np.log2(p.sum()) + xs.max()


def _case(seed=0):
    # two pieces of 3 tiles: the first holds keys that agree with the query
    # (scores near +200 in log2 units), the second keys that oppose it (near
    # -200) and a ragged last tile of 40 real keys
    rng = np.random.default_rng(seed)
    D = 8
    n1, n2 = 3 * TILE, 2 * TILE + 40
    x1 = (200.0 + rng.normal(size=n1)).astype(np.float32)
    x2 = np.zeros(3 * TILE, np.float32)
    x2[:n2] = (-200.0 + rng.normal(size=n2)).astype(np.float32)
    v1 = rng.normal(size=(n1, D)).astype(np.float32)
    v2 = np.zeros((3 * TILE, D), np.float32)
    v2[:n2] = rng.normal(size=(n2, D)).astype(np.float32)
    return (x1, v1, n1), (x2, v2, n2)


def test_unmasked_padding_flushes_an_opposing_piece():
    _, (x2, v2, n2) = _case()
    out, w = piece_frame(x2, v2, n2, mask_pad=False)
    assert not np.isfinite(out).all()          # 0/0: the real weights were flushed
    assert w == -np.inf


def test_masked_padding_matches_the_exact_piece():
    _, (x2, v2, n2) = _case()
    out, w = piece_frame(x2, v2, n2, mask_pad=True)
    ref, lse2 = _exact(x2, v2, n2)
    assert np.isfinite(out).all()
    # E4M3 weights: a few percent of relative error on the weighted mean
    assert np.abs(out - ref).max() <= 0.1 * np.abs(v2[:n2]).max()
    assert abs(w - lse2) <= 0.1


def test_combine_of_masked_pieces_matches_exact_and_unmasked_is_nan():
    (x1, v1, n1), (x2, v2, n2) = _case()
    xs = np.concatenate([x1, x2[:n2]])
    vs = np.concatenate([v1, v2[:n2]])
    ref, _ = _exact(xs, vs, len(xs))
    good = combine([piece_frame(x1, v1, n1, True), piece_frame(x2, v2, n2, True)])
    bad = combine([piece_frame(x1, v1, n1, False), piece_frame(x2, v2, n2, False)])
    assert np.abs(good - ref).max() <= 0.1 * np.abs(v1).max()
    assert not np.isfinite(bad).all()          # 0 * NaN in the combine


def test_whole_segment_of_centred_keys_is_unaffected_by_padding():
    # a whole segment: scores of centred keys average to zero, so the largest
    # real score is >= 0 and an unmasked zero never moves the reference
    rng = np.random.default_rng(1)
    n = 5 * TILE + 17
    s = rng.normal(size=n) * 3.0
    s -= s.mean()
    x = np.zeros(6 * TILE, np.float32)
    x[:n] = s
    v = np.zeros((6 * TILE, 4), np.float32)
    v[:n] = rng.normal(size=(n, 4))
    a = piece_frame(x, v, n, mask_pad=False)
    b = piece_frame(x, v, n, mask_pad=True)
    assert np.array_equal(a[0], b[0]) and a[1] == b[1]
