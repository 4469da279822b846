"""GPU parity at the largest matrix the C ABI accepts at K = 8192: 43349 tiles
of 16 rows (the last one ragged), a code plane of 2,130,690,048 bytes just
below the 2 GiB - 16 MiB that the kernels' 32-bit buffer offsets allow
(one tile more is rejected, tests/test_abi.py).  The codes (5.7 GB) are drawn
on the device from a seeded generator; sampled rows -- the first tile, rows
spread over the matrix and the last 40, in the last tile and the ones before it
-- are compared with the oracle at 1 token (vector ALUs and matrix cores), 16
and 64 tokens, |y - y_ref| <= 1e-3 * sum|x w|."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, dev

pytestmark = pytest.mark.gpu

TILES = ((1 << 31) - (1 << 24)) // (192 * 256)   # 43349 tiles of 49152 code bytes at K = 8192


@pytest.fixture(scope="module")
def q3():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_fp8_codebook_amd as q3
    q3.lib()
    return q3


def test_largest_accepted_matrix(q3):
    n, k = 16 * TILES - 7, 8192
    assert q3.q3_layout(n, k)["code_plane_bytes"] == TILES * 192 * 256 <= (1 << 31) - (1 << 24)
    codes, codebook, scales, x = synth.make_layer_on_device(n, k, 64, seed=77)
    rows = np.unique(np.r_[0:16, np.linspace(16, n - 41, 60).astype(np.int64), n - 40:n])
    host_codes = codes[torch.from_numpy(rows).to(codes.device)].cpu().numpy()
    w = q3.q3_pack(codes, dev(scales), dev(codebook))
    del codes
    torch.cuda.empty_cache()
    cp, sp = oracle.pack(host_codes, scales[rows])
    for m, fn in [(1, q3.q3_gemv), (1, q3.q3_gemm_small_m), (16, q3.q3_gemm_small_m), (64, q3.q3_gemm_small_m)]:
        y_ref, bound = oracle.linear(cp, sp, codebook[rows], len(rows), k, x[:m])
        y = fn(w, dev(x[:m]))
        assert_close(y[:, torch.from_numpy(rows).to(y.device)].cpu().numpy(), y_ref, bound,
                     f"{fn.__name__} n={n} k={k} m={m}")
        del y
