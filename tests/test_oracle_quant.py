"""Pins of the quantizer oracle (Hibana page, "Model surgery": 3-bit codes into
a per-row FP8 codebook with one 8-bit scale per 32 weights; the scale and code
rules are this project's reading, stated in oracle/q3_quant.py).  Pinned to
exact rational brute force (fractions.Fraction) for scales and codes, on
random and adversarial inputs, to the reconstruction of groups that use the
codebook's largest entry, and to the scale rule's special cases."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


def _frac_value(byte):
    v = oracle.E4M3FN_TABLE[int(byte)]
    return Fraction(float(v))


def _brute_scales(w, codebook):
    n, k = w.shape
    out = np.empty((n, k // 32), dtype=np.int64)
    for r in range(n):
        cbmax = max(abs(_frac_value(b)) for b in codebook[r])
        for g in range(k // 32):
            amax = max(abs(Fraction(float(x))) for x in w[r, 32 * g:32 * g + 32])
            out[r, g] = next((s for s in range(255) if amax <= cbmax * Fraction(2) ** (s - 127)), 254)
    return out


def _brute_codes(w, codebook, scales):
    n, k = w.shape
    out = np.empty((n, k), dtype=np.int64)
    for r in range(n):
        vals = [_frac_value(b) for b in codebook[r]]
        for c in range(k):
            sc = Fraction(2) ** (int(scales[r, c // 32]) - 127)
            x = Fraction(float(w[r, c]))
            d = [abs(x - v * sc) for v in vals]
            out[r, c] = min(range(8), key=lambda j: (d[j], j))      # smallest distance, then lowest index
    return out


def _adversarial(n=6, k=64, seed=0):
    """Weights on exact midpoints, tiny weights against large codes, zeros, and
    codebooks with +-0, repeated entries and opposite-sign pairs."""
    rng = np.random.default_rng(seed)
    w, cb = synth.make_quant(n, k, seed)
    cb[0] = [0x38, 0xB8, 0x00, 0x80, 0x38, 0x40, 0xC0, 0x30]       # 1, -1, +0, -0, 1 again, 2, -2, 0.5
    cb[1] = [0x7E, 0xFE, 0x01, 0x81, 0x44, 0x44, 0x3C, 0xBC]       # +-448, +-2^-9, 3, 3, 1.5, -1.5
    for r in (0, 1):
        vals = oracle.codebook_values(cb[r])
        e = 2.0 ** rng.integers(-5, 3)
        for c in range(k):
            a, b = rng.choice(8, 2, replace=False)
            kind = c % 4
            if kind == 0:
                w[r, c] = (vals[a] + vals[b]) / 2 * e                   # exact midpoint: a tie
            elif kind == 1:
                w[r, c] = np.float32(1e-30) * (1 if c % 8 == 1 else -1)  # tiny against large codes
            elif kind == 2:
                w[r, c] = 0.0
        w[r, 0] = np.max(np.abs(vals)) * e                               # the group fits exactly at e
    w[2, :32] = 0.0                                                     # all-zero group
    cb[3] = 0                                                           # a codebook of zeros
    return w.astype(np.float32), cb


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_matches_rational_brute_force(seed):
    w, cb = synth.make_quant(5, 96, seed)
    codes, scales = oracle.quantize(w, cb)
    assert np.array_equal(scales, _brute_scales(w, cb))
    assert np.array_equal(codes, _brute_codes(w, cb, scales))


def test_adversarial_matches_rational_brute_force():
    w, cb = _adversarial()
    codes, scales = oracle.quantize(w, cb)
    assert np.array_equal(scales, _brute_scales(w, cb))
    assert np.array_equal(codes, _brute_codes(w, cb, scales))
    assert scales[2, 0] == 0                           # all-zero group: the smallest scale
    assert np.all(scales[3] == 254)                    # nothing fits a codebook of zeros
    assert np.all(codes[3] == 0)                       # every entry is 0: the lowest index


def test_ties_go_to_the_lower_index():
    cb = np.array([[0x40, 0x38, 0x38, 0x00, 0x80, 0xB8, 0x30, 0x44]], dtype=np.uint8)   # 2, 1, 1, +0, -0, -1, .5, 3
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, :6] = [1.0, 0.0, 1.5, -0.25, 0.75, 2.5]
    w[0, 31] = 3.0                                     # group max = codebook max: scale 127
    codes, scales = oracle.quantize(w, cb)
    assert scales[0, 0] == 127
    # 1 -> index 1 (not the repeat at 2); 0 -> +0 (index 3, before -0); 1.5 is between 1 (idx 1) and 2 (idx 0):
    # equal distance -> index 0; -0.25 between 0 and -0.5? -0.5 is absent: 0 (idx 3) is nearest;
    # 0.75 is between 0.5 (idx 6) and 1 (idx 1): tie -> 1; 2.5 between 2 (idx 0) and 3 (idx 7): tie -> 0
    assert codes[0, :6].tolist() == [1, 3, 0, 3, 1, 0]
    assert codes[0, 31] == 7


def test_groups_using_the_largest_entry_reconstruct_exactly():
    layer = synth.make_layer(8, 128, seed=3)
    codes = layer.codes.copy()
    vals = oracle.codebook_values(layer.codebook)
    top = np.abs(vals).argmax(axis=1)
    codes[:, ::32] = top[:, None]                       # every group uses its row's largest entry
    w = oracle.dequantize(codes, layer.scales, layer.codebook).astype(np.float32)
    assert np.array_equal(w.astype(np.float64), oracle.dequantize(codes, layer.scales, layer.codebook))
    c2, s2 = oracle.quantize(w, layer.codebook)
    assert np.array_equal(s2, layer.scales)
    assert np.array_equal(oracle.dequantize(c2, s2, layer.codebook), w.astype(np.float64))


def test_scale_rule_edges():
    cb = np.full((1, 8), 0x38, dtype=np.uint8)           # cbmax = 1
    w = np.zeros((1, 96), dtype=np.float32)
    w[0, 0] = 1.0                                        # fits at 2^0 exactly
    w[0, 32] = np.nextafter(np.float32(1.0), np.float32(2))   # just above: needs 2^1
    w[0, 64] = 2.0 ** -140                               # below the smallest step: s = 0
    _, s = oracle.quantize(w, cb)
    assert s[0].tolist() == [127, 128, 0]
