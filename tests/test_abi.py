"""The C ABI library without a GPU: it loads, exports every entry point that
include/q3.h declares, its layout query agrees with the oracle's independent
layout, and argument validation rejects bad calls before touching HIP."""
import ctypes
import os
import re
import subprocess

import pytest

import oracle
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "q3.h")


@pytest.fixture(scope="module")
def q3lib():
    from bit_fp8_codebook_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from bit_fp8_codebook_amd import build
        build.build(verbose=False)
    return _lib.lib()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"Q3_API\s+[\w\s\*]+?\b(q3_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_symbols() == sorted(["q3_status_string", "q3_layout", "q3_pack", "q3_unpack", "q3_gemv",
                                         "q3_gemm_small_m", "q3_moe_topk", "q3_grouped_expert_gemv",
                                         "q3_layout2", "q3_pack2", "q3_unpack2", "q3_head2_scores",
                                         "q3_shortlist_workspace_bytes", "q3_shortlist", "q3_rescore_fp8",
                                         "q3_draft_head_workspace_bytes", "q3_draft_head", "q3_moe_budget_topk",
                                         "q3_moe_mlp_workspace_bytes", "q3_moe_mlp", "q3_quantize",
                                         "q3_moe_mlp_noalloc", "q3_moe_mlp_noalloc_max_bytes", "q3_fit_codebook",
                                         "q3_gemm_small_m_workspace_bytes", "q3_gemm_small_m_ws"])


def test_library_exports_every_declared_symbol(q3lib):
    from bit_fp8_codebook_amd import _lib
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT\s+(q3_\w+)", out))
    for s in declared_symbols():
        assert s in exported, s
        assert hasattr(q3lib, s)
    assert set(_lib.SIGNATURES) == set(declared_symbols())


@pytest.mark.parametrize("n,k", [(1024, 1024), (4096, 4096), (1536, 2048), (2048, 768), (28672, 8192),
                                 (151936, 4096), (5, 32), (3, 96), (7, 160), (1, 8224)])
def test_layout_matches_oracle(q3lib, n, k):
    from bit_fp8_codebook_amd import q3_layout
    got = q3_layout(n, k)
    ref = oracle.layout(n, k)
    for key in ref:
        assert got[key] == ref[key], key


@pytest.mark.parametrize("n,k", [(151936, 4096), (1024, 1024), (5, 32), (37, 160), (1, 8224)])
def test_layout2_matches_oracle(q3lib, n, k):
    from bit_fp8_codebook_amd import q3_layout2
    got = q3_layout2(n, k)
    ref = oracle.layout2(n, k)
    for key in ref:
        assert got[key] == ref[key], key


def test_workspace_sizes(q3lib):
    # shortlist scratch: 64 chunk lists of 16 (score, row) pairs per query
    assert q3lib.q3_shortlist_workspace_bytes(1) == 64 * 16 * 8
    assert q3lib.q3_shortlist_workspace_bytes(0) == 0
    # draft head: fp32 scores [m][n] (rounded up to 8 bytes), then the shortlist scratch
    assert q3lib.q3_draft_head_workspace_bytes(1, 151936) == 151936 * 4 + 64 * 16 * 8
    assert q3lib.q3_draft_head_workspace_bytes(3, 5) == 64 + 3 * 64 * 16 * 8
    # fused MLP: h (bf16, two terms per pair, I = n_gu / 2) and per-pair fp32
    # outputs (rows padded to 4), each piece 256-aligned
    assert q3lib.q3_moe_mlp_workspace_bytes(1536, 2048, 8, 8) == 2 * 64 * 768 * 2 + 64 * 2048 * 4
    assert q3lib.q3_moe_mlp_workspace_bytes(64, 30, 1, 1) == 256 + 256
    assert q3lib.q3_moe_mlp_workspace_bytes(1536, 2048, 9, 8) == 0      # more than 64 pairs
    assert q3lib.q3_moe_mlp_workspace_bytes(1504, 2048, 8, 8) == 0      # I not a multiple of 32


def test_gemm_small_m_workspace_sizes(q3lib):
    ws = q3lib.q3_gemm_small_m_workspace_bytes
    # activations staged in LDS whole (m * k up to about 68K elements): one pass, no workspace
    assert ws(4096, 4096, 8) == 0
    assert ws(4096, 4096, 16) == 0
    assert ws(96, 1024, 16) == 0
    # a wide grid needs no K split: the 28672 x 8192 verify batch and the vocabulary projection
    assert ws(28672, 8192, 16) == 0
    assert ws(151936, 4096, 64) == 0
    # few row tiles and streamed activations: fp32 partial planes, splits * m * n floats
    assert ws(4096, 8192, 16) == 8 * 16 * 4096 * 4
    assert ws(4096, 4096, 64) == 4 * 64 * 4096 * 4
    assert ws(8192, 28672, 16) == 4 * 16 * 8192 * 4
    assert ws(8192, 28672, 64) == 2 * 64 * 8192 * 4
    # 17..64 tokens on 512..1535 row tiles at K <= 4096: one pass, one row tile per wave
    assert ws(8192, 4096, 64) == 0
    assert ws(12000, 4096, 40) == 0
    assert ws(8192, 8192, 64) == 2 * 64 * 8192 * 4
    # one token on whole steps past 512 row tiles (K = 4096, 8192, up to 1536 tiles): the split-K kernel
    assert ws(24576, 8192, 1) == 0
    assert ws(24576, 4096, 1) == 0
    # invalid shapes report no workspace
    assert ws(4096, 4096, 65) == 0
    assert ws(4096, 4100, 16) == 0
    assert ws(0, 4096, 16) == 0


def test_gemm_small_m_ws_validation(q3lib):
    from bit_fp8_codebook_amd import _lib
    fake = 0x1000
    w = _lib.Q3Matrix(4096, 4096, fake, fake, fake)
    f = q3lib.q3_gemm_small_m_ws
    assert f(ctypes.byref(w), fake, 65, 4096, fake, 4096, fake, 1 << 20, None) == 2      # m > 64
    assert f(ctypes.byref(w), fake, 0, 4096, fake, 4096, fake, 1 << 20, None) == 2
    assert f(ctypes.byref(w), fake, 16, 4096, fake, 4096, fake + 4, 1 << 20, None) == 3  # workspace 16-aligned
    assert f(ctypes.byref(w), fake, 16, 4000, fake, 4096, fake, 1 << 20, None) == 1      # ldx < k
    assert f(None, fake, 16, 4096, fake, 4096, fake, 1 << 20, None) == 1


def test_head_validation_rejects_before_any_hip_call(q3lib):
    from bit_fp8_codebook_amd import _lib
    fake = 0x1000
    w2 = _lib.Q3Matrix(16, 64, fake, fake, fake)
    assert q3lib.q3_head2_scores(ctypes.byref(w2), fake, 17, 64, fake, 16, None) == 2    # m > 16
    assert q3lib.q3_head2_scores(ctypes.byref(w2), fake, 0, 64, fake, 16, None) == 2
    mis = _lib.Q3Matrix(16, 64, fake, fake, fake + 2)                                    # codebook not 4-aligned
    assert q3lib.q3_head2_scores(ctypes.byref(mis), fake, 1, 64, fake, 16, None) == 3
    assert q3lib.q3_pack2(fake, 63, fake, 2, 16, 64, fake, fake, None) == 1
    sw = q3lib.q3_shortlist_workspace_bytes(1)
    assert q3lib.q3_shortlist(fake, 1, 100, 100, 17, fake, sw, fake, None, None) == 2         # size > 16
    assert q3lib.q3_shortlist(fake, 1, 10, 10, 11, fake, sw, fake, None, None) == 2           # size > n
    assert q3lib.q3_shortlist(fake, 1, 100, 99, 16, fake, sw, fake, None, None) == 1          # ld < n
    assert q3lib.q3_shortlist(fake, 1, 100, 100, 16, fake + 4, sw, fake, None, None) == 3     # workspace 8-aligned
    assert q3lib.q3_shortlist(None, 1, 100, 100, 16, fake, sw, fake, None, None) == 1
    assert q3lib.q3_shortlist(fake, 1, 100, 100, 16, fake, sw - 8, fake, None, None) == 1     # workspace too small
    assert q3lib.q3_shortlist(fake, 2, 100, 100, 16, fake, sw, fake, None, None) == 1         # sized for 1 query
    h8 = _lib.Q3Mxfp8Matrix(16, 64, fake, 64, fake, 2)
    assert q3lib.q3_rescore_fp8(ctypes.byref(h8), fake, 1, 64, fake, 17, fake, fake, None) == 2
    h8.ld_elements = 72                                                                    # not a multiple of 16
    assert q3lib.q3_rescore_fp8(ctypes.byref(h8), fake, 1, 64, fake, 16, fake, fake, None) == 3
    h8.ld_elements = 48                                                                    # < k
    assert q3lib.q3_rescore_fp8(ctypes.byref(h8), fake, 1, 64, fake, 16, fake, fake, None) == 1
    dw = q3lib.q3_draft_head_workspace_bytes(1, 16)
    h8 = _lib.Q3Mxfp8Matrix(16, 96, fake, 96, fake, 3)                                     # k differs from w2's
    assert q3lib.q3_draft_head(ctypes.byref(w2), ctypes.byref(h8), fake, 1, 96, 16, fake, dw, fake, fake, fake,
                               None) == 1
    h8 = _lib.Q3Mxfp8Matrix(16, 64, fake, 64, fake, 2)
    assert q3lib.q3_draft_head(ctypes.byref(w2), ctypes.byref(h8), fake, 1, 64, 16, fake, dw - 8, fake, fake, fake,
                               None) == 1                                                    # workspace too small
    assert q3lib.q3_draft_head(ctypes.byref(w2), ctypes.byref(h8), fake, 2, 64, 16, fake, dw, fake, fake, fake,
                               None) == 1                                                    # sized for 1 query


def test_status_strings(q3lib):
    for s in range(6):
        assert q3lib.q3_status_string(s)


def test_validation_rejects_before_any_hip_call(q3lib):
    from bit_fp8_codebook_amd import _lib
    info = _lib.Q3LayoutInfo()
    assert q3lib.q3_layout(4, 33, ctypes.byref(info)) == 2
    assert q3lib.q3_layout(4, 0, ctypes.byref(info)) == 2
    assert q3lib.q3_layout(-1, 32, ctypes.byref(info)) == 1
    assert q3lib.q3_layout(4, 32, None) == 1
    fake = 0x1000   # never dereferenced: every call below fails validation first
    w = _lib.Q3Matrix(16, 64, fake, fake, fake)
    assert q3lib.q3_gemv(None, fake, 1, 64, fake, 16, None) == 1
    assert q3lib.q3_gemv(ctypes.byref(w), fake, 0, 64, fake, 16, None) == 2       # m = 0
    assert q3lib.q3_gemv(ctypes.byref(w), fake, 9, 64, fake, 16, None) == 2       # m > 8
    assert q3lib.q3_gemm_small_m(ctypes.byref(w), fake, 65, 64, fake, 16, None) == 2
    assert q3lib.q3_gemv(ctypes.byref(w), None, 1, 64, fake, 16, None) == 1       # null x
    assert q3lib.q3_gemv(ctypes.byref(w), fake + 2, 1, 64, fake, 16, None) == 3   # x misaligned
    assert q3lib.q3_gemv(ctypes.byref(w), fake, 1, 60, fake, 16, None) == 1       # ldx < k
    assert q3lib.q3_gemv(ctypes.byref(w), fake, 1, 64, fake, 8, None) == 1        # ldy < n
    bad = _lib.Q3Matrix(16, 48, fake, fake, fake)                                  # k % 32 != 0
    assert q3lib.q3_gemv(ctypes.byref(bad), fake, 1, 64, fake, 16, None) == 2
    mis = _lib.Q3Matrix(16, 64, fake + 4, fake, fake)                              # code plane not 16-aligned
    assert q3lib.q3_gemv(ctypes.byref(mis), fake, 1, 64, fake, 16, None) == 3
    mis = _lib.Q3Matrix(16, 64, fake, fake + 2, fake)                              # scale plane not 4-aligned
    assert q3lib.q3_gemv(ctypes.byref(mis), fake, 1, 64, fake, 16, None) == 3
    huge = _lib.Q3Matrix(1 << 20, 8192, fake, fake, fake)                          # code plane >= 2 GiB
    assert q3lib.q3_gemv(ctypes.byref(huge), fake, 1, 8192, fake, 1 << 20, None) == 2
    # one 16-row tile past the largest accepted K = 8192 matrix (43349 tiles of 49152 code bytes stay
    # below 2 GiB - 16 MiB; 43350 do not): rejected (tests/test_gpu_limits.py runs the largest one)
    over = _lib.Q3Matrix(16 * 43349 + 1, 8192, fake, fake, fake)
    assert q3lib.q3_gemv(ctypes.byref(over), fake, 1, 8192, fake, 16 * 43349 + 1, None) == 2
    assert q3lib.q3_gemm_small_m(ctypes.byref(over), fake, 16, 8192, fake, 16 * 43349 + 1, None) == 2
    nul = _lib.Q3Matrix(16, 64, fake, None, fake)
    assert q3lib.q3_gemv(ctypes.byref(nul), fake, 1, 64, fake, 16, None) == 1
    assert q3lib.q3_pack(fake, 63, fake, 2, 16, 64, fake, fake, None) == 1        # ldc < k
    assert q3lib.q3_pack(fake, 64, fake, 1, 16, 64, fake, fake, None) == 1        # lds < k/32
    assert q3lib.q3_pack(fake, 64, fake, 2, 16, 64, fake + 8, fake, None) == 3
    assert q3lib.q3_moe_topk(fake, 8, 64, 65, fake, None) == 2
    assert q3lib.q3_moe_topk(fake, 8, 2048, 8, fake, None) == 2
    assert q3lib.q3_moe_budget_topk(fake, 8, 64, 8, 7, fake, None, None) == 2     # budget < topk
    assert q3lib.q3_moe_budget_topk(fake, 8, 64, 8, 65, fake, None, None) == 2    # budget > experts
    assert q3lib.q3_moe_budget_topk(fake, 1025, 64, 8, 16, fake, None, None) == 2  # too many tokens
    assert q3lib.q3_moe_budget_topk(fake, 8, 64, 8, 16, fake, fake + 2, None) == 3
    assert q3lib.q3_moe_budget_topk(None, 8, 64, 8, 16, fake, None, None) == 1
    # n = 16, k = 64: one tile of 192*4 = 768 code bytes and 64 scale bytes.
    st = _lib.Q3ExpertStack(4, 16, 64, fake, 768, fake, 64, fake, 128)
    assert q3lib.q3_grouped_expert_gemv(ctypes.byref(st), fake, 64, 2, fake, 8, 8, fake, 16, None) == 1
    assert q3lib.q3_grouped_expert_gemv(ctypes.byref(st), fake, 64, 0, fake, 9, 8, fake, 16, None) == 2
    st.code_expert_stride = 752                                                     # smaller than a plane
    assert q3lib.q3_grouped_expert_gemv(ctypes.byref(st), fake, 64, 0, fake, 8, 8, fake, 16, None) == 1
    st.code_expert_stride = 776                                                     # not 16-aligned
    assert q3lib.q3_grouped_expert_gemv(ctypes.byref(st), fake, 64, 0, fake, 8, 8, fake, 16, None) == 3
    # codebook fitting
    assert q3lib.q3_fit_codebook(fake, 64, 4, 48, fake, None) == 2            # k % 32 != 0
    assert q3lib.q3_fit_codebook(fake, 1 << 19, 4, 1 << 19, fake, None) == 2  # k above 2^18
    assert q3lib.q3_fit_codebook(fake, 60, 4, 64, fake, None) == 1            # ldw < k
    assert q3lib.q3_fit_codebook(fake + 4, 64, 4, 64, fake, None) == 3        # w not 16-aligned
    assert q3lib.q3_fit_codebook(fake, 66, 4, 64, fake, None) == 3            # ldw % 4
    assert q3lib.q3_fit_codebook(fake, 64, 4, 64, fake + 4, None) == 3        # codebook not 8-aligned
    assert q3lib.q3_fit_codebook(None, 64, 4, 64, fake, None) == 1
    # quantizer
    assert q3lib.q3_quantize(fake, 64, fake, 4, 48, fake, 64, fake, 2, None) == 2       # k % 32 != 0
    assert q3lib.q3_quantize(fake, 60, fake, 4, 64, fake, 64, fake, 2, None) == 1       # ldw < k
    assert q3lib.q3_quantize(fake, 64, fake, 4, 64, fake, 64, fake, 1, None) == 1       # lds < k/32
    assert q3lib.q3_quantize(fake + 4, 64, fake, 4, 64, fake, 64, fake, 2, None) == 3   # w not 16-aligned
    assert q3lib.q3_quantize(fake, 66, fake, 4, 64, fake, 64, fake, 2, None) == 3       # ldw % 4
    assert q3lib.q3_quantize(fake, 64, fake + 4, 4, 64, fake, 64, fake, 2, None) == 3   # codebook not 8-aligned
    assert q3lib.q3_quantize(fake, 64, fake, 4, 64, fake + 4, 64, fake, 2, None) == 3   # codes not 8-aligned
    assert q3lib.q3_quantize(fake, 64, fake, 4, 64, fake, 68, fake, 2, None) == 3       # ldc % 8
    assert q3lib.q3_quantize(None, 64, fake, 4, 64, fake, 64, fake, 2, None) == 1
    # fused MLP: gate/up n = 64 (I = 32), k = 64; down n = 16, k = 32
    gu = _lib.Q3ExpertStack(4, 64, 64, fake, 3072, fake, 256, fake, 512)
    dn = _lib.Q3ExpertStack(4, 16, 32, fake, 768, fake, 64, fake, 128)
    ws = q3lib.q3_moe_mlp_workspace_bytes(64, 16, 2, 2)
    mlp = lambda g, d, t=2, topk=2, logits=fake, wsp=fake, wsb=ws: q3lib.q3_moe_mlp(
        ctypes.byref(g), ctypes.byref(d), fake, 64, fake, t, topk, logits, 4, wsp, wsb, fake, 16, None)
    assert mlp(gu, dn, logits=None) == 1
    assert mlp(gu, dn, t=33) == 2                                                   # 66 pairs
    assert mlp(gu, dn, wsb=ws - 1) == 1                                             # workspace too small
    assert mlp(gu, dn, wsp=fake + 16) == 3                                          # workspace not 256-aligned
    dn.k = 64
    assert mlp(gu, dn) == 2                                                         # down k != I
    dn.k, dn.num_experts = 32, 3
    assert mlp(gu, dn) == 1                                                         # expert counts differ


def test_binding_rejects_outputs_of_the_wrong_shape():
    # A caller-supplied output goes to the library as a pointer and a row pitch,
    # so the binding must see exactly the shape the call writes: a y with fewer
    # rows than tokens would be written past its end.
    import torch
    from bit_fp8_codebook_amd import _lib
    ok = torch.empty((3, 10), dtype=torch.float32)
    assert _lib._out(ok, 3, 10, "cpu") is ok
    assert _lib._out(torch.empty((8, 12), dtype=torch.float32)[:3, :10], 3, 10, "cpu") is not None  # strided rows
    for bad in (torch.empty((2, 10), dtype=torch.float32),          # short: 2 rows for 3 tokens
                torch.empty((3, 9), dtype=torch.float32),           # narrow
                torch.empty((3, 10), dtype=torch.float64),          # wrong type
                torch.empty((10, 3), dtype=torch.float32).t(),      # columns not contiguous
                torch.empty((30,), dtype=torch.float32)):           # flat
        with pytest.raises(ValueError):
            _lib._out(bad, 3, 10, "cpu")
    with pytest.raises(ValueError):
        _lib._check_out(torch.empty((4, 7), dtype=torch.int32), (4, 8), torch.int32, "cpu", "ids")
    with pytest.raises(ValueError):
        _lib._check_out(torch.empty(15, dtype=torch.int32), (16,), torch.int32, "cpu", "experts")
    with pytest.raises(ValueError):
        _lib._check_out(torch.empty((4, 64), dtype=torch.uint8), (4, 2), torch.uint8, "cpu", "scales")
    with pytest.raises(ValueError):
        _lib._workspace(torch.empty((4, 8), dtype=torch.uint8)[:, :4], "cpu")        # not contiguous
    assert _lib._nbytes(torch.empty(10, dtype=torch.float32)) == 40


def test_noalloc_mlp_validation(q3lib):
    # The library's scratch holds 4 MiB per GPU; rounds whose intermediate
    # buffers need more are rejected on the host, before any HIP call.
    from bit_fp8_codebook_amd import _lib
    assert q3lib.q3_moe_mlp_noalloc_max_bytes() == 4 << 20
    fake = 0x1000
    # 64 pairs need 256 * (I + ceil(n_down / 4) * 4) bytes: I = 8192 with n_down = 8192 fits exactly.
    gu = _lib.Q3ExpertStack(4, 2 * 8192, 64, fake, 1 << 30, fake, 1 << 26, fake, 1 << 20)
    dn = _lib.Q3ExpertStack(4, 8192, 8192, fake, 1 << 30, fake, 1 << 26, fake, 1 << 20)
    assert q3lib.q3_moe_mlp_workspace_bytes(2 * 8192, 8192, 8, 8) == 4 << 20
    call = lambda g, d, t=8, topk=8, logits=fake: q3lib.q3_moe_mlp_noalloc(
        ctypes.byref(g), ctypes.byref(d), fake, 64, fake, t, topk, logits, 4, fake, 8200, None)
    assert call(gu, dn, logits=None) == 1
    assert call(gu, dn, t=9) == 2                                                   # 72 pairs
    dn.n = 8193                                                                      # one more output row
    assert call(gu, dn) == 2                                                        # exceeds the scratch
    dn.n, dn.k = 8192, 4096
    assert call(gu, dn) == 2                                                        # down k != I
