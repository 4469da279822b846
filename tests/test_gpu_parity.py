"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.  Packing and unpacking must be bit-exact; products must
satisfy |y - y_ref| <= 1e-3 * sum_k |x_k w_k| for every output."""
import numpy as np
import pytest
import torch

import oracle
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


PACK_SHAPES = [(1024, 1024), (37, 96), (5, 32), (64, 160), (2048, 768), (100, 4096), (3, 8224)]


@pytest.mark.parametrize("n,k", PACK_SHAPES)
def test_pack_bit_exact(q3, n, k):
    layer = synth.make_layer(n, k, seed=n + k)
    rng = np.random.default_rng(k)
    codes = layer.codes | (rng.integers(0, 32, size=layer.codes.shape, dtype=np.uint8) << 3)  # high bits ignored
    w = q3.q3_pack(dev(codes), dev(layer.scales), dev(layer.codebook))
    cp, sp = oracle.pack(codes, layer.scales)
    assert np.array_equal(w.code_plane.cpu().numpy(), cp)
    assert np.array_equal(w.scale_plane.cpu().numpy(), sp)
    c2, s2 = q3.q3_unpack(w)
    assert np.array_equal(c2.cpu().numpy(), codes & 7)
    assert np.array_equal(s2.cpu().numpy(), layer.scales)


def test_pack_worked_example(q3):
    codes = np.array([[k % 8 for k in range(32)]], dtype=np.uint8)
    w = q3.q3_pack(dev(codes), dev(np.array([[127]], dtype=np.uint8)), dev(np.zeros((1, 8), np.uint8)))
    plane = w.code_plane.cpu().numpy()
    # k = 32, one row: one quad per step, so word j is the first word of piece 16*j (byte 256*j).
    words = [int(plane[256 * j:256 * j + 4].view(np.uint32)[0]) for j in range(3)]
    assert [hex(v) for v in words] == ["0xfbb26920", "0xbb32a920", "0xfbf2a9a0"]
    assert w.scale_plane.cpu().numpy()[0] == 127


GEMV_CASES = [(1024, 1024, 1), (4096, 4096, 1), (4096, 4096, 4), (4096, 4096, 8), (37, 96, 3), (1, 32, 1),
              (130, 800, 2), (1000, 768, 5), (257, 8224, 6), (2048, 2048, 7), (300, 1536, 8), (64, 8192, 1)]


@pytest.mark.parametrize("n,k,m", GEMV_CASES)
def test_gemv_parity(q3, n, k, m):
    layer, x = synth.make_linear(n, k, m, seed=n * 7 + k + m)
    w = pack_layer(q3, layer)
    y = q3.q3_gemv(w, dev(x)).cpu().numpy()
    y_ref, bound = oracle_linear(layer, x)
    assert_close(y, y_ref, bound, f"gemv n={n} k={k} m={m}")


MFMA_CASES = [(1024, 1024, 1), (4096, 4096, 1), (4096, 4096, 4), (4096, 4096, 8), (4096, 4096, 16),
              (100, 96, 3), (17, 32, 16), (333, 1024, 17), (200, 768, 33), (513, 2048, 64), (64, 8224, 5),
              (2000, 8192, 16), (48, 4096, 48), (77, 2048, 40), (250, 4096, 24), (1290, 3072, 64),
              (300, 2080, 64)]


@pytest.mark.parametrize("n,k,m", MFMA_CASES)
def test_gemm_small_m_parity(q3, n, k, m):
    layer, x = synth.make_linear(n, k, m, seed=n * 11 + k + m)
    w = pack_layer(q3, layer)
    y = q3.q3_gemm_small_m(w, dev(x)).cpu().numpy()
    y_ref, bound = oracle_linear(layer, x)
    assert_close(y, y_ref, bound, f"gemm n={n} k={k} m={m}")


@pytest.mark.parametrize("fn", ["q3_gemv", "q3_gemm_small_m"])
def test_strided_x_and_y(q3, fn):
    layer, x = synth.make_linear(70, 512, 4, seed=3)
    w = pack_layer(q3, layer)
    xbig = torch.zeros((4, 512 + 64), dtype=torch.int16, device="cuda")
    xbig[:, :512] = dev(x)
    ybig = torch.full((4, 70 + 5), 7.0, dtype=torch.float32, device="cuda")
    getattr(q3, fn)(w, xbig[:, :512], ybig[:, :70])
    yb = ybig.cpu().numpy()
    assert np.all(yb[:, 70:] == 7.0)
    y_ref, bound = oracle_linear(layer, x)
    assert_close(yb[:, :70], y_ref, bound, fn)


@pytest.mark.parametrize("m", [16, 64])
def test_aligned_y_ragged_rows(q3, m):
    # y rows 16-byte aligned (four outputs per store) with a row count that ends
    # inside a group of four: the last outputs go out one by one, the pad stays.
    n, k = 1290, 2048
    layer, x = synth.make_linear(n, k, m, seed=m + 1)
    w = pack_layer(q3, layer)
    ybig = torch.full((m, n + 6), 7.0, dtype=torch.float32, device="cuda")
    q3.q3_gemm_small_m(w, dev(x), ybig[:, :n])
    yb = ybig.cpu().numpy()
    assert np.all(yb[:, n:] == 7.0)
    y_ref, bound = oracle_linear(layer, x)
    assert_close(yb[:, :n], y_ref, bound, f"aligned y m={m}")


@pytest.mark.parametrize("fn,m", [("q3_gemv", 1), ("q3_gemv", 8), ("q3_gemm_small_m", 16), ("q3_gemm_small_m", 64)])
def test_deterministic(q3, fn, m):
    layer, x = synth.make_linear(1024, 4096, m, seed=5)
    w = pack_layer(q3, layer)
    xd = dev(x)
    a = getattr(q3, fn)(w, xd).cpu().numpy()
    b = getattr(q3, fn)(w, xd).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_edge_values(q3):
    """Codebooks with -0, repeated and extreme entries; scales at the ends of the
    supported range; a row whose codebook is all zero (bound 0 -> exact 0)."""
    layer, x = synth.make_linear(64, 256, 3, seed=8)
    layer.codebook[0, :] = 0x00
    layer.codebook[1, :] = 0x80
    layer.codebook[2, :] = 0x7E            # 448
    layer.codebook[3, :] = 0xFE            # -448
    layer.codebook[4, :] = 0x01            # 2^-9
    layer.codebook[5, ::2] = 0x38
    layer.scales[6, :] = 16
    layer.scales[7, :] = 240
    layer.scales[8, :] = np.array([16, 240, 127, 100, 150, 16, 240, 127], dtype=np.uint8)
    w = pack_layer(q3, layer)
    y_ref, bound = oracle_linear(layer, x)
    for fn in ("q3_gemv", "q3_gemm_small_m"):
        y = getattr(q3, fn)(w, dev(x)).cpu().numpy()
        assert_close(y, y_ref, bound, fn)
        assert np.all(y[:, :2] == 0)


@pytest.mark.parametrize("n,k,m", [(64, 256, 1), (64, 256, 4), (9000, 512, 1), (9000, 512, 16), (9000, 512, 64)])
def test_subnormal_activations(q3, n, k, m):
    """bf16 activations in the subnormal range (exponent field 0, random sign
    and mantissa), mixed with zeros and one normal token row when m > 1,
    against weights scaled by 2^13: every exact product stays in fp32's normal
    range, so the bound holds only if the conversions and products keep the
    subnormal inputs rather than flush them.  The shapes reach the split-K
    kernel (vector ALUs and matrix cores), the tall and full-K kernels past 512
    row tiles, and the wide kernel at 64 tokens."""
    layer, _ = synth.make_linear(n, k, 1, seed=31)
    layer.scales[:] = 140
    rng = np.random.default_rng(31)
    x = (rng.integers(1, 128, size=(m, k)) | (rng.integers(0, 2, size=(m, k)) << 15)).astype(np.uint16)
    x[0, ::7] = 0
    if m > 1:
        x[1] = synth.make_linear(1, k, 1, seed=32)[1][0]     # a normal row next to the subnormal ones
    w = pack_layer(q3, layer)
    y_ref, bound = oracle_linear(layer, x)
    assert np.all(bound[0] > 2.0 ** -126)
    for fn in ("q3_gemv", "q3_gemm_small_m") if m <= 8 else ("q3_gemm_small_m",):
        y = getattr(q3, fn)(w, dev(x)).cpu().numpy()
        assert_close(y, y_ref, bound, f"{fn} n={n} k={k} m={m}")


def test_empty_matrix(q3):
    layer, x = synth.make_linear(0, 64, 1, seed=1)
    w = q3.empty_packed(0, 64, "cuda")
    y = torch.empty((1, 0), dtype=torch.float32, device="cuda")
    q3.q3_gemv(w, dev(x), y)
    q3.q3_gemm_small_m(w, dev(x), y)


def test_device_side_rejections(q3):
    layer, x = synth.make_linear(16, 64, 9, seed=2)
    w = pack_layer(q3, layer)
    with pytest.raises(q3.Q3Error, match="UNSUPPORTED_SHAPE"):
        q3.q3_gemv(w, dev(x))
    xd = torch.zeros((1, 72), dtype=torch.int16, device="cuda")
    with pytest.raises(q3.Q3Error, match="MISALIGNED"):
        q3.q3_gemv(w, xd[:, 1:65])


# --------------------------------------------------------------- full sizes

def test_config3_full_size_all_rows(q3):
    """K=8192, N=28672, M=16 (batched verify): every output against the oracle."""
    layer, x = synth.make_linear(28672, 8192, 16, seed=0)
    w = pack_layer(q3, layer)
    y = q3.q3_gemm_small_m(w, dev(x)).cpu().numpy()
    del w
    y_ref, bound = oracle_linear(layer, x)
    assert_close(y, y_ref, bound, "config 3")


def test_config4_full_size_all_rows(q3):
    """K=4096, N=151936, M=64 (vocabulary projection, fp32 logits): every output
    against the oracle (computed in row blocks on the host)."""
    layer, x = synth.make_linear(151936, 4096, 64, seed=0)
    w = pack_layer(q3, layer)
    y = q3.q3_gemm_small_m(w, dev(x)).cpu().numpy()
    del w
    torch.cuda.empty_cache()
    y_ref, bound = oracle_linear(layer, x)
    assert_close(y, y_ref, bound, "config 4")


@pytest.mark.parametrize("n,k,m", [(90000, 1024, 64), (90000, 1536, 40), (90000, 2048, 33)])
def test_many_row_groups_all_rows(q3, n, k, m):
    # The wide kernel on a tall matrix with 2, 3 and 4 steps of 512 k (the odd
    # count ends on the step after its paired loop), several blocks per CU and
    # a last row group that is only partly inside the matrix.
    layer, x = synth.make_linear(n, k, m, seed=k + m)
    w = pack_layer(q3, layer)
    y = q3.q3_gemm_small_m(w, dev(x)).cpu().numpy()
    y_ref, bound = oracle_linear(layer, x)
    assert_close(y, y_ref, bound, f"n={n} k={k} m={m}")


@pytest.mark.parametrize("n,k,m", [(128005, 2560, 64), (128005, 2048, 40), (151936, 2560, 33)])
def test_halfstep_wide_all_rows(q3, n, k, m):
    # Vocabulary-sized matrices with three or four column tiles take the wide
    # kernel's half-step variant (two blocks per CU): a ragged last row tile
    # (its tiles past n re-read the last one), an odd step count, and column
    # tiles only partly filled with tokens.
    layer, x = synth.make_linear(n, k, m, seed=n + k + m)
    w = pack_layer(q3, layer)
    y = q3.q3_gemm_small_m(w, dev(x)).cpu().numpy()
    del w
    y_ref, bound = oracle_linear(layer, x)
    assert_close(y, y_ref, bound, f"half-step wide n={n} k={k} m={m}")


def test_halfstep_wide_strided_x_and_y(q3):
    # The half-step kernel with activation rows 64 elements apart beyond K and
    # output rows whose stride keeps them from 16-byte alignment (one store per
    # output), the pad around both left untouched.
    n, k, m = 128005, 2048, 40
    layer, x = synth.make_linear(n, k, m, seed=77)
    w = pack_layer(q3, layer)
    xbig = torch.zeros((m, k + 64), dtype=torch.int16, device="cuda")
    xbig[:, :k] = dev(x)
    ybig = torch.full((m, n + 3), 7.0, dtype=torch.float32, device="cuda")
    q3.q3_gemm_small_m(w, xbig[:, :k], ybig[:, :n])
    del w
    yb = ybig.cpu().numpy()
    assert np.all(yb[:, n:] == 7.0)
    y_ref, bound = oracle_linear(layer, x)
    assert_close(yb[:, :n], y_ref, bound, "half-step wide, strided x and y")


@pytest.mark.parametrize("m", [1, 4, 8])
def test_config1_full_gemv_and_mfma(q3, m):
    layer, x = synth.make_linear(4096, 4096, m, seed=0)
    w = pack_layer(q3, layer)
    y_ref, bound = oracle_linear(layer, x)
    assert_close(q3.q3_gemv(w, dev(x)).cpu().numpy(), y_ref, bound, "gemv config 1")
    assert_close(q3.q3_gemm_small_m(w, dev(x)).cpu().numpy(), y_ref, bound, "mfma config 1")
