"""Pins of the codebook-fitting oracle (oracle/q3_fit.py) against facts fixed
independently of its code: math.frexp for the group exponents, exact Fraction
arithmetic for the grid, torch's float8_e4m3fn conversion and a brute force
over all finite E4M3FN values for the final rounding, a brute-force Fraction
recomputation of every Lloyd update, the fixed-point property at convergence,
the non-increasing sum of squared errors, and exact recovery of a row built
from eight values."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import q3_fit


def _rng(seed):
    return np.random.default_rng(seed)


def test_group_exponents_match_frexp():
    rng = _rng(1)
    w = (rng.standard_normal((3, 256)) * np.exp2(rng.integers(-140, 60, (3, 256)))).astype(np.float32)
    w[0, :32] = 0.0                                  # all-zero group
    w[1, 32:64] = 0.0
    w[1, 40] = 0.5                                   # exact power of two: e = -1
    w[2, 64:96] = np.float32(2.0 ** -140)            # subnormal fp32
    w[2, 96:128] = -np.float32(1.5 * 2 ** 20)
    e = q3_fit.group_exponents(w)
    for r in range(3):
        for g in range(8):
            m = max(abs(float(v)) for v in w[r, 32 * g:32 * g + 32])
            if m == 0:
                assert e[r, g] == 0
                continue
            f, x = math.frexp(m)
            want = x - 1 if f == 0.5 else x
            assert e[r, g] == want
            assert m <= 2.0 ** e[r, g] and not m <= 2.0 ** (e[r, g] - 1)


def test_grid_values_are_exact_rounding_half_even():
    rng = _rng(2)
    w = (rng.standard_normal((2, 64)) * 3).astype(np.float32)
    # exact halves of the grid step in group 0: ties must go to even
    w[0, 0] = np.float32(2.5 / 4096 * 4)             # group max forces e below
    w[0, 1:32] = 0
    w[0, 1] = np.float32(3.0)                        # max 3 -> e = 2, step 2^-10
    w[0, 2] = np.float32(2.5 * 2 ** -10)             # 2.5 steps -> 2
    w[0, 3] = np.float32(3.5 * 2 ** -10)             # 3.5 steps -> 4
    w[0, 4] = np.float32(-2.5 * 2 ** -10)            # -2.5 -> -2
    q = q3_fit.grid_values(w)
    e = q3_fit.group_exponents(w)
    for r in range(2):
        for k in range(64):
            exact = Fraction(float(w[r, k])) * Fraction(2) ** (12 - int(e[r, k // 32]))
            assert q[r, k] == round(exact)           # Python rounds Fractions half to even
    assert q[0, 2] == 2 and q[0, 3] == 4 and q[0, 4] == -2
    assert np.abs(q).max() <= 4096


def _torch_e4m3(values):
    t = torch.tensor([float(v) for v in values], dtype=torch.float64).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_rounding_matches_torch_on_dyadic_values():
    rng = _rng(3)
    vals = []
    for _ in range(2000):
        s = int(rng.integers(-(1 << 20), 1 << 20))          # |value| <= 256: inside E4M3FN's range
        c = 1 << int(rng.integers(0, 10))
        vals.append(Fraction(s, c * 4096))
    # exact midpoints between neighbouring E4M3FN values (ties to even), both signs
    pos = [v for _, v in q3_fit.E4M3FN_POSITIVE]
    for a, b in zip(pos[:-1], pos[1:]):
        if b <= 1:
            vals += [(a + b) / 2, -(a + b) / 2]
    got = np.array([q3_fit.round_e4m3fn(v) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, _torch_e4m3(vals))


def test_e4m3_rounding_brute_force_on_rationals():
    rng = _rng(4)
    for _ in range(300):
        v = Fraction(int(rng.integers(-(1 << 20), 1 << 20)), int(rng.integers(1, 5000)) * 4096)
        b = q3_fit.round_e4m3fn(v)
        mag = Fraction(0) if (b & 0x7F) == 0 else dict(q3_fit.E4M3FN_POSITIVE)[b & 0x7F]
        d = abs(abs(v) - mag)
        for bb, vv in q3_fit.E4M3FN_POSITIVE:      # nothing strictly nearer
            assert abs(abs(v) - vv) >= d
        assert (b >> 7) == (1 if v < 0 else 0)


def _brute_update(q, cents):
    """One Lloyd update in plain Fractions: nearest (ties to lower index),
    exact means, empty clusters keep their value, stable sort by value."""
    cv = [Fraction(s, c) for s, c in cents]
    members = [[] for _ in cents]
    for x in q:
        d = [abs(int(x) - c) for c in cv]
        members[d.index(min(d))].append(int(x))
    new = [(sum(m), len(m)) if m else cents[j] for j, m in enumerate(members)]
    order = sorted(range(len(new)), key=lambda j: (Fraction(*new[j]), j))
    return [new[j] for j in order]


def test_nearest_equal_distances_go_to_the_lower_centroid():
    # Grid values exactly midway between two centroids, integer and rational
    # (9/2 and 11/2 around 5), checked against exact Fraction distances with
    # the lower index taken on equal distances.
    cents = [(-8, 1), (0, 1), (2, 1), (9, 2), (11, 2), (20, 3), (10, 1), (60, 1)]
    q = np.array([-4, 1, 5, 8, 3, 6, 35, 61, -9, 0, 2], dtype=np.int64)
    got = q3_fit.nearest(q, cents)
    cv = [Fraction(sn, c) for sn, c in cents]
    for x, j in zip(q.tolist(), got.tolist()):
        d = [abs(x - c) for c in cv]
        assert j == d.index(min(d)), (x, j)
    # hand-derived: -4 ties -8/0 -> 0; 1 ties 0/2 -> 1; 5 ties 9/2 and 11/2 -> 3;
    # 8 is nearest 20/3 -> 5; 35 ties 10/60 -> 6
    assert got.tolist()[:4] == [0, 1, 3, 5] and got[6] == 6


def _sse(q, cents):
    cv = [Fraction(s, c) for s, c in cents]
    return sum(min((int(x) - c) ** 2 for c in cv) for x in q)


@pytest.mark.parametrize("seed,K", [(5, 32), (6, 96), (7, 256), (8, 64)])
def test_lloyd_updates_match_brute_force(seed, K):
    rng = _rng(seed)
    q = rng.integers(-4096, 4097, K).astype(np.int64)
    if seed == 8:
        q = rng.integers(-3, 4, K).astype(np.int64)   # few distinct values: equal centroids, empty clusters
    trace = []
    final = q3_fit.lloyd(q, trace)
    prev = q3_fit.initial_centroids(q)
    srt = sorted(int(v) for v in q)
    assert prev == [(srt[(2 * i + 1) * K // 16], 1) for i in range(8)]
    sse = [_sse(q, prev)]
    for step in trace:
        assert [Fraction(*c) for c in step] == [Fraction(*c) for c in _brute_update(q, prev)]
        sse.append(_sse(q, step))
        prev = step
    assert all(b <= a for a, b in zip(sse, sse[1:])), "Lloyd updates never increase the squared error"
    assert final == trace[-1]
    if len(trace) < q3_fit.MAX_UPDATES:
        # converged: a fixed point -- every cluster's centroid is its mean
        assert [Fraction(*c) for c in _brute_update(q, final)] == [Fraction(*c) for c in final]


def test_eight_values_repeated_are_recovered_exactly():
    vals = np.array([-1.0, -0.5, -0.25, -0.125, 0.125, 0.375, 0.75, 1.0], dtype=np.float32)
    w = np.tile(vals, 4)[None, :].copy()             # K = 32, each value 4 times, group max 1 -> e = 0
    _rng(9).shuffle(w[0])
    cb = q3_fit.fit_codebook(w)[0]
    want = torch.tensor(vals.astype(np.float64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(cb, want)


def test_zero_row_and_shapes():
    assert np.array_equal(q3_fit.fit_codebook(np.zeros((2, 64), np.float32)), np.zeros((2, 8), np.uint8))
    with pytest.raises(ValueError):
        q3_fit.fit_codebook(np.zeros((2, 48), np.float32))


def test_fitted_codebook_is_sorted_and_beats_a_fixed_one():
    # On N(0,1) rows the fitted codebook (then the quantizer's scales and codes)
    # reconstructs better than a fixed symmetric codebook: a sanity check that
    # the fit serves its purpose, not a parity pin.
    import oracle
    rng = _rng(10)
    w = rng.standard_normal((4, 1024)).astype(np.float32)
    cb = q3_fit.fit_codebook(w)
    vals = oracle.codebook_values(cb)
    assert np.all(np.diff(vals, axis=1) >= 0)
    fixed = np.tile(torch.tensor([-1.0, -0.6, -0.3, -0.1, 0.1, 0.3, 0.6, 1.0], dtype=torch.float64)
                    .to(torch.float8_e4m3fn).view(torch.uint8).numpy(), (4, 1))

    def err(cbk):
        codes, scales = oracle.quantize(w, cbk)
        rec = np.take_along_axis(oracle.codebook_values(cbk), codes.astype(np.int64), axis=1)
        rec = rec * np.exp2(np.repeat(scales.astype(np.int64) - 127, 32, axis=1))
        return float(((rec - w) ** 2).sum())
    assert err(cb) < err(fixed)
