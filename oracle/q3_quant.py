"""Oracle of the quantizer (test infrastructure only: tests, the smoke check and
the CPU baseline use it; the GPU product path never imports it).

Hibana page, "Model surgery": each group of 32 weights of a row is stored as
3-bit indices into the row's 8-entry FP8 codebook plus one 8-bit scale.  The
page does not say how a weight matrix is brought to that form.  Readings taken
(for a given per-row codebook; fitting the codebook needs trained weights and
is not part of this step):

  scale   s[r][g] = the smallest s in 0..254 with
              max_{k in group g} |w[r][k]| <= max_j |cb_r[j]| * 2^(s - 127),
          i.e. the group's largest magnitude just fits the codebook's largest
          magnitude (no clipping); 254 when no s fits (a codebook of zeros).
          An all-zero group gets s = 0.
  code    c[r][k] = argmin_j |w[r][k] - cb_r[j] * 2^(s[r][g] - 127)|, equal
          distances (and equal codebook values) to the lower index j.

Both are exact decisions.  The distance comparison is done without rounding:
for candidates a and b, |w - b| < |w - a| exactly when (a - b) and
(2w - a - b) have opposite signs ((w-b)^2 - (w-a)^2 = (a-b)(2w-a-b)); a + b
and 2w are exact in float64 for these operands, and the sign of a rounded
difference is the sign of the exact one.

Inputs: w float32 [n][k] (finite, |w| <= 2^64), k % 32 == 0; codebook uint8
E4M3FN [n][8] without NaN entries.

Pins (tests/test_oracle_quant.py): brute force in exact rational arithmetic
(fractions.Fraction) for the scale and for every code on adversarial inputs
(exact midpoints, tiny weights against large codes, +-0 entries, repeated
entries, opposite-sign pairs), the reconstruction of any group that uses the
codebook's largest entry, and the special cases of the scale rule.
"""
from __future__ import annotations

import numpy as np

from .q3_oracle import E4M3FN_TABLE

GROUP = 32


def codebook_values(codebook: np.ndarray) -> np.ndarray:
    """E4M3FN bytes [n][8] -> float64 values."""
    return E4M3FN_TABLE[np.asarray(codebook, dtype=np.int64)]


def choose_scales(w: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """Scale byte of every group (reading above), by trying every s from the top."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    amax = np.abs(w.astype(np.float64)).reshape(n, k // GROUP, GROUP).max(axis=2)   # [n][G]
    cbmax = np.abs(codebook_values(codebook)).max(axis=1)[:, None]                   # [n][1]
    s = np.full(amax.shape, 254, dtype=np.int64)
    for cand in range(254, -1, -1):          # ends on the smallest s that fits
        fits = amax <= np.ldexp(cbmax, cand - 127)
        s = np.where(fits, cand, s)
    return s.astype(np.uint8)


def snap(w: np.ndarray, codebook: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Nearest code of every weight under its group's scale (reading above)."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    G = k // GROUP
    e = np.asarray(scales, dtype=np.int64).astype(np.int32) - 127                     # [n][G]
    v = np.ldexp(codebook_values(codebook)[:, None, :], e[:, :, None])                # [n][G][8], exact
    ww = w.astype(np.float64).reshape(n, G, GROUP)
    best = np.zeros(ww.shape, dtype=np.int64)
    a = np.broadcast_to(v[:, :, :1], ww.shape)                                        # value of the best so far
    for j in range(1, 8):
        b = np.broadcast_to(v[:, :, j:j + 1], ww.shape)
        t = 2.0 * ww - (a + b)
        closer = np.where(a > b, t < 0, np.where(a < b, t > 0, False))               # |w-b| < |w-a|
        best = np.where(closer, j, best)
        a = np.where(closer, b, a)
    return best.reshape(n, k).astype(np.uint8)


def quantize(w: np.ndarray, codebook: np.ndarray):
    """(codes uint8 [n][k], scales uint8 [n][k/32]) of w under the given codebooks."""
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % GROUP or w.shape[1] == 0:
        raise ValueError("w must be [n][k] with k a positive multiple of 32")
    scales = choose_scales(w, codebook)
    return snap(w, codebook, scales), scales
