"""GPU parity of the split-K products on matrices with few row tiles (one
block per 16-row tile, K dealt out to up to 16 waves in half-steps of 8 groups
per quad): every output against the oracle, |y - y_ref| <= 1e-3 * sum|x w|.

The cases span every wave count (2, 4, 8, 16 waves: K = 32..4096), two
half-steps per wave (K above 4096, up to 8 tokens), one token with whole
steps per wave (K from 3072 up, with waves past the last step; up to 1536
row tiles at K = 4096 and 8192, and the first matrices past each limit), last steps holding 1, 2
or 3 quads (K % 512 != 0), ragged row counts, the 512-tile boundary (the next
matrix takes the earlier kernels), 1..16 tokens on the matrix cores and one
to four tokens on the vector ALUs, strided and unaligned operands, run-to-run
determinism and graph replays."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_close, dev, oracle_linear, pack_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q3():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_fp8_codebook_amd as q3
    q3.lib()
    return q3


# (n, k, m): waves per tile follow from K (half-steps = 2 * ceil(K / 512)).
CASES = [
    (16, 32, 1), (37, 96, 3), (5, 160, 16),              # one step, 1 quad (2 waves)
    (130, 800, 2), (1000, 768, 5), (64, 1024, 16),       # two steps, partial second (4 waves)
    (333, 1056, 7), (2048, 2048, 1), (2048, 2048, 9),    # 8 waves; K = 1056 ends on a 1-quad step
    (2048, 2048, 4), (1000, 1056, 4), (130, 800, 3), (4096, 4096, 3),   # 3 and 4 tokens on the vector ALUs
    (4096, 4096, 1), (4096, 4096, 2), (4096, 4096, 4), (4095, 4096, 8), (4096, 4096, 12), (4096, 4096, 16),
    (100, 4000, 15),                                      # 16 waves, last step of 3 quads
    (4096, 8192, 1), (1000, 8192, 8), (300, 6176, 4),    # two half-steps per wave
    (8192, 4096, 1), (8192, 4096, 16),                    # 512 tiles: the largest the kernel takes
    (8193, 4096, 1),                                      # 513 tiles: earlier kernels
    (1, 4096, 1), (17, 4096, 16),
    # one token on the matrix cores, whole steps per wave (K >= 3072, K % 512 == 0)
    (3000, 3072, 1), (2048, 4096, 1), (4608, 4096, 1), (5000, 6144, 1), (100, 8192, 1), (17, 5120, 1),
    (3584, 4096, 1), (4097, 4096, 1),                     # 224 and 257 tiles: either side of the half-step range
    # one token, whole steps, past 512 tiles (K = 4096 or 8192, up to 1536 tiles)
    (11008, 4096, 1), (16385, 4096, 1), (24576, 4096, 1), (24577, 4096, 1), (12288, 8192, 1), (9000, 6144, 1),
    (16400, 8192, 1), (24576, 8192, 1),                   # K = 8192 past 1024 tiles: two steps per wave
]


@pytest.mark.parametrize("n,k,m", CASES)
def test_splitk_parity(q3, n, k, m):
    layer, x = synth.make_linear(n, k, m, seed=5 * n + k + m)
    w = pack_layer(q3, layer)
    xd = dev(x)
    y_ref, bound = oracle_linear(layer, x)
    assert_close(q3.q3_gemm_small_m(w, xd).cpu().numpy(), y_ref, bound, f"matrix cores n={n} k={k} m={m}")
    if m <= 8:
        assert_close(q3.q3_gemv(w, xd).cpu().numpy(), y_ref, bound, f"vector ALUs n={n} k={k} m={m}")


@pytest.mark.parametrize("m,k", [(1, 4096), (3, 4096), (16, 4096), (1, 3072)])
def test_splitk_strided_and_unaligned(q3, m, k):
    # x rows 4160 elements apart; y rows 4101 floats apart starting one float
    # into the buffer, so outputs leave one by one.  K = 3072 at one token
    # takes whole steps per wave.
    n = 4096
    layer, x = synth.make_linear(n, k, m, seed=40 + m)
    w = pack_layer(q3, layer)
    xbig = torch.zeros((m, 4160), dtype=torch.int16, device="cuda")
    xbig[:, :k] = dev(x)
    ybuf = torch.full((m * 4101 + 1,), float("nan"), dtype=torch.float32, device="cuda")
    y = ybuf[1:].view(m, 4101)[:, :n]
    y_ref, bound = oracle_linear(layer, x)
    q3.q3_gemm_small_m(w, xbig[:, :k], y)
    assert_close(y.cpu().numpy(), y_ref, bound, f"strided m={m}")
    pad = ybuf[1:].view(m, 4101)[:, n:].cpu().numpy()
    assert np.all(np.isnan(pad)), "bytes past each output row must stay untouched"
    assert np.isnan(ybuf[0].item())
    if m == 1:
        y.fill_(float("nan"))
        q3.q3_gemv(w, xbig[:, :k], y)
        assert_close(y.cpu().numpy(), y_ref, bound, "strided gemv")


def test_splitk_deterministic(q3):
    layer, x = synth.make_linear(4096, 4096, 16, seed=91)
    w = pack_layer(q3, layer)
    xd = dev(x)
    a = q3.q3_gemm_small_m(w, xd).cpu().numpy()
    b = q3.q3_gemm_small_m(w, xd).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    g1 = q3.q3_gemv(w, xd[:1]).cpu().numpy()
    g2 = q3.q3_gemv(w, xd[:1]).cpu().numpy()
    assert np.array_equal(g1.view(np.uint32), g2.view(np.uint32))
    # one token, whole steps per wave
    layer, x = synth.make_linear(2048, 8192, 1, seed=92)
    w = pack_layer(q3, layer)
    xd = dev(x)
    f1 = q3.q3_gemm_small_m(w, xd).cpu().numpy()
    f2 = q3.q3_gemm_small_m(w, xd).cpu().numpy()
    assert np.array_equal(f1.view(np.uint32), f2.view(np.uint32))


def test_splitk_needs_no_workspace(q3):
    # The workspace entry point reports no workspace for shapes this kernel takes.
    assert q3.q3_gemm_small_m_workspace_bytes(4096, 4096, 16) == 0
    assert q3.q3_gemm_small_m_workspace_bytes(4096, 8192, 8) == 0
    assert q3.q3_gemm_small_m_workspace_bytes(24576, 8192, 1) == 0      # whole steps past 512 tiles
    layer, x = synth.make_linear(2048, 2048, 6, seed=3)
    w = pack_layer(q3, layer)
    y_ref, bound = oracle_linear(layer, x)
    assert_close(q3.q3_gemm_small_m_ws(w, dev(x)).cpu().numpy(), y_ref, bound, "workspace entry point")


def test_splitk_graph_replays(q3):
    """Captured in a graph, every replay (with eager work between) equals the eager result."""
    layer, x = synth.make_linear(4096, 4096, 1, seed=17)
    w = pack_layer(q3, layer)
    xd = dev(x)
    eager_g = q3.q3_gemv(w, xd).cpu().numpy()
    eager_m = q3.q3_gemm_small_m(w, xd).cpu().numpy()
    yg = torch.zeros((1, 4096), dtype=torch.float32, device="cuda")
    ym = torch.zeros((1, 4096), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        q3.q3_gemv(w, xd, yg)
        q3.q3_gemm_small_m(w, xd, ym)
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            q3.q3_gemv(w, xd, yg)
            q3.q3_gemm_small_m(w, xd, ym)
    torch.cuda.synchronize()
    for _ in range(3):
        yg.zero_()
        ym.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(yg.cpu().numpy(), eager_g)
        assert np.array_equal(ym.cpu().numpy(), eager_m)
        q3.q3_gemv(w, xd)                       # eager work between replays
        torch.cuda.synchronize()
