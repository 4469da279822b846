"""GPU parity of the workspace variant of the matrix-core product
(q3_gemm_small_m_ws): when the activations are streamed and the matrix has few
16-row tiles, K is split over blocks into fp32 partial planes that a second
launch adds in split order.  Every case is checked against the CPU oracle with
|y - y_ref| <= 1e-3 * sum_k |x_k w_k|, and against the one-pass product."""
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


def splits_of(q3, n, k, m):
    b = q3.q3_gemm_small_m_workspace_bytes(n, k, m)
    return b // (4 * m * n) if b else 1


# (n, k, m): verify batches on 4096 rows (the 8-wave stream kernel for m <= 16
# at K = 8192, the wide kernel with two row tiles per wave for m > 16), a
# ragged matrix whose groups per row are not a multiple of 16 (stream kernel
# with 3 column tiles), a small ragged one, and a K that leaves a partial last
# step.
FULL = [(4096, 8192, 12), (4096, 8192, 16), (4096, 4096, 33), (4096, 4096, 64), (1000, 4128, 40),
        (520, 6176, 17), (300, 6176, 16)]


@pytest.mark.parametrize("n,k,m", FULL)
def test_split_parity_full(q3, n, k, m):
    assert splits_of(q3, n, k, m) > 1, "case must exercise the K split"
    layer, x = synth.make_linear(n, k, m, seed=n + k + m)
    w = pack_layer(q3, layer)
    xd = dev(x)
    y_ref, bound = oracle_linear(layer, x)
    y_ws = q3.q3_gemm_small_m_ws(w, xd).cpu().numpy()
    assert_close(y_ws, y_ref, bound, f"split n={n} k={k} m={m}")
    assert_close(q3.q3_gemm_small_m(w, xd).cpu().numpy(), y_ref, bound, f"one pass n={n} k={k} m={m}")


@pytest.mark.parametrize("n,k,m", [(8192, 28672, 16), (8192, 28672, 64)])
def test_split_parity_down_projection_sampled_rows(q3, n, k, m):
    """The down-projection shape (K = 28672, N = 8192): few row tiles, long K."""
    assert splits_of(q3, n, k, m) > 1
    layer, x = synth.make_linear(n, k, m, seed=m)
    w = pack_layer(q3, layer)
    y = q3.q3_gemm_small_m_ws(w, dev(x)).cpu().numpy()
    rows = np.sort(np.concatenate([np.random.default_rng(m).choice(n, 120, replace=False), [0, 15, 16, n - 1]]))
    y_ref, bound = oracle_linear(layer, x, rows=rows)
    assert_close(y[:, rows], y_ref, bound, f"down projection m={m}")
    # the one-pass product (no workspace) on the same shape
    y1 = q3.q3_gemm_small_m(w, dev(x)).cpu().numpy()
    assert_close(y1[:, rows], y_ref, bound, f"down projection one pass m={m}")


@pytest.mark.parametrize("n,k,m", [(1000, 9216, 8), (520, 24576, 3), (4096, 28672, 4)])
def test_vector_alu_streamed_activations(q3, n, k, m):
    """q3_gemv with activations too large to stage whole in LDS (streamed one
    512-k step at a time), on matrices with few row tiles."""
    layer, x = synth.make_linear(n, k, m, seed=7 * n + m)
    w = pack_layer(q3, layer)
    y_ref, bound = oracle_linear(layer, x)
    assert_close(q3.q3_gemv(w, dev(x)).cpu().numpy(), y_ref, bound, f"gemv streamed n={n} k={k} m={m}")


def test_split_deterministic_and_workspace_contents_irrelevant(q3):
    n, k, m = 4096, 4096, 64
    layer, x = synth.make_linear(n, k, m, seed=11)
    w = pack_layer(q3, layer)
    xd = dev(x)
    nbytes = q3.q3_gemm_small_m_workspace_bytes(n, k, m)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a = q3.q3_gemm_small_m_ws(w, xd, workspace=ws).cpu().numpy()
    ws.fill_(0xFF)   # NaN bit patterns everywhere: every partial must be overwritten
    b = q3.q3_gemm_small_m_ws(w, xd, workspace=ws).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_small_workspace_falls_back_to_one_pass(q3):
    n, k, m = 4096, 8192, 16
    layer, x = synth.make_linear(n, k, m, seed=12)
    w = pack_layer(q3, layer)
    xd = dev(x)
    nbytes = q3.q3_gemm_small_m_workspace_bytes(n, k, m)
    small = torch.zeros(nbytes - 16, dtype=torch.uint8, device="cuda")
    y_small = q3.q3_gemm_small_m_ws(w, xd, workspace=small).cpu().numpy()
    y_plain = q3.q3_gemm_small_m(w, xd).cpu().numpy()
    assert np.array_equal(y_small.view(np.uint32), y_plain.view(np.uint32))
    assert np.all(small.cpu().numpy() == 0), "a too-small workspace must not be written"


def test_split_strided_unaligned_y(q3):
    # y rows not 16-byte aligned and padded: the reduce stores one by one and
    # leaves the pad alone; x rows strided.
    n, k, m = 1001, 4096, 20
    assert splits_of(q3, n, k, m) > 1
    layer, x = synth.make_linear(n, k, m, seed=13)
    w = pack_layer(q3, layer)
    xbig = torch.zeros((m, k + 64), dtype=torch.int16, device="cuda")
    xbig[:, :k] = dev(x)
    ybig = torch.full((m, n + 4), 7.0, dtype=torch.float32, device="cuda")
    q3.q3_gemm_small_m_ws(w, xbig[:, :k], ybig[:, 1:n + 1])
    yb = ybig.cpu().numpy()
    assert np.all(yb[:, 0] == 7.0) and np.all(yb[:, n + 1:] == 7.0)
    y_ref, bound = oracle_linear(layer, x)
    assert_close(yb[:, 1:n + 1], y_ref, bound, "strided split")


def test_split_graph_replays(q3):
    n, k, m = 4096, 4096, 32
    layer, x = synth.make_linear(n, k, m, seed=14)
    w = pack_layer(q3, layer)
    xd = dev(x)
    ws = torch.empty(q3.q3_gemm_small_m_workspace_bytes(n, k, m), dtype=torch.uint8, device="cuda")
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    eager = q3.q3_gemm_small_m_ws(w, xd, workspace=ws).cpu().numpy()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        q3.q3_gemm_small_m_ws(w, xd, y, ws)
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            q3.q3_gemm_small_m_ws(w, xd, y, ws)
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(float(rep))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), eager.view(np.uint32)), f"replay {rep}"


@pytest.mark.parametrize("n,k,m,split", [(65536, 2048, 40, False), (65536, 2048, 20, False),
                                         (33600, 4096, 64, True), (33600, 4096, 40, True)])
def test_wide_five_row_tiles_sampled_rows(q3, n, k, m, split):
    """The wide kernel with five row tiles per wave at 2..4 column tiles, on its
    own and with K split over blocks (a matrix whose five-tile grid has fewer
    than 128 blocks but would gain nothing from two-tile blocks)."""
    assert (splits_of(q3, n, k, m) > 1) == split
    layer, x = synth.make_linear(n, k, m, seed=n + m)
    w = pack_layer(q3, layer)
    y = (q3.q3_gemm_small_m_ws(w, dev(x)) if split else q3.q3_gemm_small_m(w, dev(x))).cpu().numpy()
    rng = np.random.default_rng(m)
    rows = np.sort(np.concatenate([rng.choice(n, 120, replace=False), [0, 15, 16, 319, 320, n - 1]]))
    y_ref, bound = oracle_linear(layer, x, rows=rows)
    assert_close(y[:, rows], y_ref, bound, f"n={n} k={k} m={m}")


@pytest.mark.parametrize("n,k,m", [(8192, 4096, 64), (12000, 4096, 40), (20000, 2048, 17)])
def test_wide_one_row_tile_per_wave(q3, n, k, m):
    """512..1535 row tiles at K <= 4096 with 17..64 tokens: one row tile per wave
    of the wide kernel, in one pass through both entry points (sampled rows)."""
    assert splits_of(q3, n, k, m) == 1
    layer, x = synth.make_linear(n, k, m, seed=3 * n + m)
    w = pack_layer(q3, layer)
    xd = dev(x)
    rows = np.sort(np.concatenate([np.random.default_rng(n).choice(n, 200, replace=False), [0, 15, 16, n - 1]]))
    y_ref, bound = oracle_linear(layer, x, rows=rows)
    assert_close(q3.q3_gemm_small_m(w, xd).cpu().numpy()[:, rows], y_ref, bound, f"one pass n={n} k={k} m={m}")
    assert_close(q3.q3_gemm_small_m_ws(w, xd).cpu().numpy()[:, rows], y_ref, bound, f"workspace n={n} k={k} m={m}")

