"""GPU parity of per-row codebook fitting (q3_fit_codebook; the procedure is the
reading stated in include/q3.h and oracle/q3_fit.py): codebook bytes bit-exact
against the oracle on seeded rows (N(0,1) weights with a power of two per
group), adversarial rows (few distinct values, ties on grid midpoints, equal
centroids and empty clusters, all-zero groups and rows, subnormal and very
large weights, one group), the longest rows taken (2^18), strided operands,
rows of the K=8192 N=28672 matrix, and fit -> quantize against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q3():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_fp8_codebook_amd as q3
    q3.lib()
    return q3


def _fit(q3, w):
    return q3.q3_fit_codebook(torch.from_numpy(np.ascontiguousarray(w)).cuda()).cpu().numpy()


@pytest.mark.parametrize("n,k", [(64, 1024), (17, 8192), (5, 32), (33, 96), (40, 4128), (3, 65536)])
def test_fit_bit_exact(q3, n, k):
    w, _ = synth.make_quant(n, k, seed=3 * n + k)
    assert np.array_equal(_fit(q3, w), oracle.fit_codebook(w))


def _adversarial_rows():
    rng = np.random.default_rng(77)
    rows = []
    rows.append(np.zeros(256, np.float32))                                       # all zero
    r = rng.standard_normal(256).astype(np.float32)
    r[32:96] = 0                                                                  # zero groups
    rows.append(r)
    rows.append(np.full(256, 0.75, np.float32))                                   # one value
    rows.append(np.tile(np.array([1, -1], np.float32), 128))                      # two values
    rows.append(rng.integers(-3, 4, 256).astype(np.float32))                      # 7 values: equal starts
    rows.append((rng.integers(-4096, 4097, 256) * 2.0 ** -12).astype(np.float32))  # on the grid
    r = (rng.integers(-8192, 8193, 256) * 2.0 ** -13).astype(np.float32)
    r[::32] = 1.0                                                                 # half-steps of the grid: ties
    rows.append(r)
    rows.append((rng.standard_normal(256) * 2.0 ** -140).astype(np.float32))      # subnormal weights
    rows.append((rng.standard_normal(256) * 2.0 ** 60).astype(np.float32))        # very large weights
    r = rng.standard_normal(256).astype(np.float32)
    r[::2] *= np.float32(2.0 ** -30)                                              # dynamic range inside groups
    rows.append(r)
    rows.append(np.tile(np.array([-1, -0.5, -0.25, -0.125, 0.125, 0.375, 0.75, 1.0], np.float32), 32))
    rows.append(-np.abs(rng.standard_normal(256)).astype(np.float32) * 1e-3)     # all negative, tiny centroids
    return np.stack(rows)


def test_fit_adversarial(q3):
    w = _adversarial_rows()
    assert np.array_equal(_fit(q3, w), oracle.fit_codebook(w))


def test_fit_one_group_and_longest_rows(q3):
    w, _ = synth.make_quant(7, 32, seed=8)
    assert np.array_equal(_fit(q3, w), oracle.fit_codebook(w))
    w, _ = synth.make_quant(2, 1 << 18, seed=9)
    assert np.array_equal(_fit(q3, w), oracle.fit_codebook(w))


def test_fit_strided(q3):
    w, _ = synth.make_quant(20, 512, seed=10)
    big = torch.full((20, 600), float("nan"), dtype=torch.float32, device="cuda")   # padding never read
    big[:, :512] = torch.from_numpy(w).cuda()
    cb = torch.full((20, 8), 0xAB, dtype=torch.uint8, device="cuda")
    q3.q3_fit_codebook(big[:, :512], cb)
    assert np.array_equal(cb.cpu().numpy(), oracle.fit_codebook(w))


def test_fit_full_matrix_sampled_rows(q3):
    """K=8192, N=28672: every row fitted on the GPU, 384 rows checked."""
    n, k = 28672, 8192
    gen = torch.Generator(device="cuda").manual_seed(0)
    w = torch.randn((n, k), generator=gen, device="cuda", dtype=torch.float32)
    cb = q3.q3_fit_codebook(w).cpu().numpy()
    rows = np.sort(np.concatenate([np.random.default_rng(1).choice(n, 380, replace=False), [0, 1, n - 2, n - 1]]))
    wr = w[torch.from_numpy(rows).cuda()].cpu().numpy()
    assert np.array_equal(cb[rows], oracle.fit_codebook(wr))


def test_fit_then_quantize(q3):
    w, _ = synth.make_quant(48, 2048, seed=11)
    wd = torch.from_numpy(w).cuda()
    cb = q3.q3_fit_codebook(wd)
    codes, scales = q3.q3_quantize(wd, cb)
    want_cb = oracle.fit_codebook(w)
    want_c, want_s = oracle.quantize(w, want_cb)
    assert np.array_equal(cb.cpu().numpy(), want_cb)
    assert np.array_equal(scales.cpu().numpy(), want_s)
    assert np.array_equal(codes.cpu().numpy(), want_c)
