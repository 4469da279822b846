"""Oracle of per-row codebook fitting (test infrastructure only: the tests, the
smoke check and the benchmark's CPU-baseline leg may use it; the GPU product
path never imports it).  It shares no code with the GPU path.

Hibana page, "Model surgery" / "Three-bit weights": each weight is a 3-bit
index into an 8-entry FP8 codebook, and the page's illustration fits that
codebook to the weights it serves.  The page gives no fitting procedure.
Reading taken (one codebook per output row, as for the layer; every step an
exact decision, so a GPU implementation can reproduce it bit for bit):

  1. Normalise each group of 32 by a power of two: e_g = the smallest integer
     with max_{k in g} |w_k| <= 2^e_g (e_g = 0 for an all-zero group), so the
     normalised values w_k / 2^e_g lie in [-1, 1].
  2. Put them on the grid 2^-12: q_k = round(w_k * 2^(12 - e_g)), ties to
     even (exact: scaling by a power of two, then rounding), |q_k| <= 4096.
  3. Run 1-D k-means (Lloyd) with 8 centroids on the row's K integers q_k:
       start  centroid i = the value of rank floor((2i+1) K / 16) in the
              sorted q (0-based ranks), i = 0..7;
       assign each q to its nearest centroid (smallest |q - c|), equal
              distances to the lower index;
       update each centroid with points to the exact mean of its points (a
              rational sum/count); a centroid without points keeps its value;
              then order the centroids by value (stable: equal values keep
              their index order);
       stop   when an update leaves every centroid unchanged, or after 64
              updates.
  4. Codebook entry i = centroid i / 2^12 rounded to the nearest E4M3FN value,
     ties to the even significand; the sign is the sign of the centroid's sum
     (a negative centroid that rounds to zero gives -0).

The fitted codebook then feeds the quantizer (oracle/q3_quant.py: the group
scale and the nearest code under that codebook).

Pins (tests/test_oracle_fit.py): the exponent rule against math.frexp; the grid
rounding against exact Fraction arithmetic; the E4M3FN rounding against
torch's float8_e4m3fn conversion (dyadic values, which convert exactly) and
against a Fraction brute force over all 253 finite values (ties included); the
Lloyd step against a brute-force Fraction recomputation of nearest centroids
and cluster means, the fixed-point property at convergence, the
non-increasing sum of squared errors over the updates, and the exact recovery
of a row made of 8 values repeated equally often.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

GROUP = 32
GRID_BITS = 12
GRID = 1 << GRID_BITS
CENTROIDS = 8
MAX_UPDATES = 64


def group_exponents(w: np.ndarray) -> np.ndarray:
    """e_g [n][G]: the smallest integer with max |w| of the group <= 2^e_g (0 for all-zero groups)."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    n, k = w.shape
    amax = np.abs(w).reshape(n, k // GROUP, GROUP).max(axis=2)
    f, x = np.frexp(amax)                      # amax = f * 2^x, f in [0.5, 1)
    e = np.where(f == 0.5, x - 1, x)
    return np.where(amax == 0, 0, e).astype(np.int64)


def grid_values(w: np.ndarray) -> np.ndarray:
    """q [n][k] int64: w * 2^(12 - e_g) rounded to the nearest integer, ties to even."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    n, k = w.shape
    e = np.repeat(group_exponents(w), GROUP, axis=1)
    return np.rint(np.ldexp(w, GRID_BITS - e)).astype(np.int64)   # exact in float64


def nearest(q: np.ndarray, cents) -> np.ndarray:
    """Index of the nearest centroid of every q (equal distances: lower index).
    cents: list of (sum, count) with count > 0; |q - s/c| is compared exactly
    as |q*c - s| / c, cross-multiplied in int64 (|q| <= 4096, counts <= 2^18,
    |sums| <= 2^30: products below 2^50)."""
    best = np.zeros(q.shape, dtype=np.int64)
    bs = np.full(q.shape, cents[0][0], dtype=np.int64)
    bc = np.full(q.shape, cents[0][1], dtype=np.int64)
    for j in range(1, len(cents)):
        s, c = cents[j]
        closer = np.abs(q * c - s) * bc < np.abs(q * bc - bs) * c     # strictly nearer than the best so far
        best = np.where(closer, j, best)
        bs = np.where(closer, s, bs)
        bc = np.where(closer, c, bc)
    return best


def initial_centroids(q: np.ndarray):
    srt = np.sort(q)
    K = srt.size
    return [(int(srt[(2 * i + 1) * K // 16]), 1) for i in range(CENTROIDS)]


def lloyd(q: np.ndarray, trace=None):
    """Centroids (sum, count) of one row's grid values after the updates of
    step 3; trace (a list) receives the centroids after every update."""
    q = np.asarray(q, dtype=np.int64)
    cents = initial_centroids(q)
    for _ in range(MAX_UPDATES):
        idx = nearest(q, cents)
        new = []
        for j in range(CENTROIDS):
            pts = q[idx == j]
            new.append((int(pts.sum()), int(pts.size)) if pts.size else cents[j])
        # order by value, stable (equal values keep their index order)
        new = [new[j] for j in sorted(range(CENTROIDS), key=lambda j: (Fraction(*new[j]), j))]
        if trace is not None:
            trace.append(list(new))
        same = all(Fraction(*a) == Fraction(*b) for a, b in zip(new, cents))
        cents = new
        if same:
            break
    return cents


def _e4m3fn_finite():
    """(byte, value) of every finite non-negative E4M3FN value, ascending."""
    out = []
    for b in range(0x7F):                     # 0x7F is NaN
        e, m = b >> 3, b & 7
        v = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        out.append((b, v))
    return out


E4M3FN_POSITIVE = _e4m3fn_finite()


def round_e4m3fn(value: Fraction) -> int:
    """The E4M3FN byte nearest to an exact value (|value| <= 448), equal
    distances to the even significand; the sign bit is the value's sign."""
    mag = abs(value)
    best = None
    for b, v in E4M3FN_POSITIVE:
        d = abs(mag - v)
        if best is None or d < best[0] or (d == best[0] and (b & 1) == 0):
            best = (d, b)
    return best[1] | (0x80 if value < 0 else 0)


def fit_row(w_row: np.ndarray) -> np.ndarray:
    """Codebook bytes [8] of one row of fp32 weights."""
    q = grid_values(np.asarray(w_row, dtype=np.float32)[None, :])[0]
    cents = lloyd(q)
    return np.array([round_e4m3fn(Fraction(s, c * GRID)) for s, c in cents], dtype=np.uint8)


def fit_codebook(w: np.ndarray) -> np.ndarray:
    """Fitted codebooks uint8 [n][8] (E4M3FN) of fp32 weights [n][k], k % 32 == 0, k <= 2^18."""
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % GROUP or w.shape[1] == 0 or w.shape[1] > (1 << 18):
        raise ValueError("w must be [n][k] with k a positive multiple of 32, at most 2^18")
    return np.stack([fit_row(row) for row in w]) if w.shape[0] else np.zeros((0, 8), np.uint8)
