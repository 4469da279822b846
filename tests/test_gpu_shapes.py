"""GPU parity over seeded random shapes: ragged n, k any multiple of 32 (steps
of 512 k partly filled), 1..64 tokens.  Together they reach every launch plan
of the products (activations staged whole or streamed, the wide kernel with
two or five row tiles per wave, K split over blocks or not, the vector-ALU
path up to 8 tokens); each case is checked on sampled rows against the CPU
oracle, through both the one-pass and the workspace entry points."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_close, dev, oracle_linear, pack_layer

pytestmark = pytest.mark.gpu


def random_shapes(count=24, seed=2026, max_weights=48_000_000):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        m = int(rng.integers(1, 65))
        k = 32 * int(rng.integers(1, 400))
        n = int(rng.integers(1, 40000))
        if n * k <= max_weights:
            out.append((n, k, m))
    return out


@pytest.fixture(scope="module")
def q3():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_fp8_codebook_amd as q3
    q3.lib()
    return q3


@pytest.mark.parametrize("n,k,m", random_shapes())
def test_random_shape_parity(q3, n, k, m):
    layer, x = synth.make_linear(n, k, m, seed=n + 7 * k + m)
    w = pack_layer(q3, layer)
    xd = dev(x)
    rng = np.random.default_rng(n)
    rows = np.unique(np.concatenate([rng.choice(n, min(n, 60), replace=False), [0, min(15, n - 1), n - 1],
                                     [r for r in (16, 319, 320) if r < n]]))
    y_ref, bound = oracle_linear(layer, x, rows=rows)
    y1 = q3.q3_gemm_small_m(w, xd).cpu().numpy()
    assert_close(y1[:, rows], y_ref, bound, f"one pass n={n} k={k} m={m}")
    y2 = q3.q3_gemm_small_m_ws(w, xd).cpu().numpy()
    assert_close(y2[:, rows], y_ref, bound, f"workspace n={n} k={k} m={m}")
    if m <= 8:
        y3 = q3.q3_gemv(w, xd).cpu().numpy()
        assert_close(y3[:, rows], y_ref, bound, f"vector ALU n={n} k={k} m={m}")
