"""GPU parity of the quantizer (Hibana page, "Model surgery"; the scale and code
rules are the reading stated in include/q3.h): codes and scale bytes bit-exact
against the oracle on seeded and adversarial inputs, strided operands, the
K=8192 N=28672 matrix on sampled rows, and quantize-then-pack against the
oracle's planes."""
import numpy as np
import pytest
import torch

import oracle
import synth
from test_oracle_quant import _adversarial

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q3():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_fp8_codebook_amd as q3
    q3.lib()
    return q3


def _gpu(q3, w, cb):
    codes, scales = q3.q3_quantize(torch.from_numpy(w).cuda(), torch.from_numpy(cb).cuda())
    return codes.cpu().numpy(), scales.cpu().numpy()


@pytest.mark.parametrize("n,k", [(37, 96), (4096, 4096), (5, 32), (300, 2080), (1, 8192), (64, 64)])
def test_quantize_bit_exact(q3, n, k):
    w, cb = synth.make_quant(n, k, seed=n + k)
    codes, scales = _gpu(q3, w, cb)
    want_c, want_s = oracle.quantize(w, cb)
    assert np.array_equal(scales, want_s)
    assert np.array_equal(codes, want_c)


def test_quantize_adversarial(q3):
    """Exact midpoints, tiny weights against large codes, zeros, +-0 and repeated
    entries, an all-zero group, a codebook of zeros, subnormal candidates."""
    w, cb = _adversarial(n=8, k=96, seed=4)
    w[4, 32:64] = np.float32(2.0 ** -140) * np.arange(32, dtype=np.float32)   # a group with scale 0
    codes, scales = _gpu(q3, w, cb)
    want_c, want_s = oracle.quantize(w, cb)
    assert np.array_equal(scales, want_s)
    assert np.array_equal(codes, want_c)
    assert want_s[4, 1] == 0


def test_quantize_strided(q3):
    w, cb = synth.make_quant(50, 320, seed=9)
    big = np.zeros((50, 400), dtype=np.float32)
    big[:, :320] = w
    wt = torch.from_numpy(big).cuda()[:, :320]
    codes = torch.full((50, 344), 0xEE, dtype=torch.uint8, device="cuda")
    scales = torch.full((50, 13), 0xEE, dtype=torch.uint8, device="cuda")
    q3.q3_quantize(wt, torch.from_numpy(cb).cuda(), codes[:, :320], scales[:, :10])
    want_c, want_s = oracle.quantize(w, cb)
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(c[:, :320], want_c) and np.all(c[:, 320:] == 0xEE)
    assert np.array_equal(s[:, :10], want_s) and np.all(s[:, 10:] == 0xEE)


def test_quantize_full_size_sampled_rows(q3):
    """K = 8192, N = 28672 (all 235M weights quantized in one launch), checked on 300 rows."""
    n, k = 28672, 8192
    w, cb = synth.make_quant(n, k, seed=1)
    codes, scales = q3.q3_quantize(torch.from_numpy(w).cuda(), torch.from_numpy(cb).cuda())
    rows = np.sort(np.concatenate([np.random.default_rng(3).choice(n, 298, replace=False), [0, n - 1]]))
    want_c, want_s = oracle.quantize(w[rows], cb[rows])
    assert np.array_equal(scales.cpu().numpy()[rows], want_s)
    assert np.array_equal(codes.cpu().numpy()[rows], want_c)


def test_quantize_then_pack_matches_oracle_planes(q3):
    n, k = 100, 1056
    w, cb = synth.make_quant(n, k, seed=5)
    codes, scales = q3.q3_quantize(torch.from_numpy(w).cuda(), torch.from_numpy(cb).cuda())
    packed = q3.q3_pack(codes, scales, torch.from_numpy(cb).cuda())
    want_c, want_s = oracle.quantize(w, cb)
    cp, sp = oracle.pack(want_c, want_s)
    assert np.array_equal(packed.code_plane.cpu().numpy(), cp)
    assert np.array_equal(packed.scale_plane.cpu().numpy(), sp)
