"""Pins of the two-bit draft-head oracle (a 2-bit candidate list, the choice on FP8 weights)
against facts fixed independently of its own code: the 2.25 bits/weight
count, hand-derived words and offsets, torch's FP8/bf16 decoders and fp64
matmul, exact rational brute force, and brute-force ranking."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden

GOLD = read_golden("head_format.txt")


def _rows(tag):
    return [r.split(None, 1)[1] for r in GOLD if r.split()[0] == tag]


def _group_codes(name):
    c = [0] * 32
    if name == "onehot21":
        c[21] = 3
    elif name == "halves":
        c = [1] * 16 + [2] * 16
    elif name == "eighths":
        c = [(k // 8) % 4 for k in range(32)]
    return c


@pytest.mark.parametrize("n,k", [(1, 32), (100, 4096), (151936, 4096), (37, 160)])
def test_bits_per_weight(n, k):
    L = oracle.layout2(n, k)
    assert L["payload_bytes"] * 32 == n * k * 9          # 2 + 8/32 = 2.25 bits per weight
    assert L["codebook_bytes"] == 4 * n


def test_group_words_hand_derived():
    seen = 0
    for row in _rows("group"):
        name, rest = row.split(":", 1)
        words = rest.split("->")[1].split()
        c = _group_codes(name.strip())
        assert oracle.pack_group2(c) == tuple(int(w, 16) for w in words)
        assert oracle.unpack_group2(oracle.pack_group2(c)) == c
        seen += 1
    assert seen == 3


def test_group_round_trip_brute_force():
    rng = np.random.default_rng(0)
    for _ in range(200):
        c = list(rng.integers(0, 4, 32))
        assert oracle.unpack_group2(oracle.pack_group2(c)) == c
    # every single-code change touches exactly one 2-bit field
    for k in range(32):
        for v in range(1, 4):
            c = [0] * 32
            c[k] = v
            w0, w1 = oracle.pack_group2(c)
            assert bin(w0).count("1") + bin(w1).count("1") == bin(v).count("1")


def test_offsets_hand_derived():
    for row in _rows("offset"):
        k, r, g, j, off = (int(v) for v in row.split())
        assert int(oracle.word_offset2(k, r, g, j)) == off


@pytest.mark.parametrize("n,k", [(37, 160), (16, 512), (20, 544)])
def test_every_plane_byte_owned_once(n, k):
    L = oracle.layout2(n, k)
    gp = L["padded_groups"]
    rows = np.arange(-(-n // 16) * 16)[:, None, None, None]
    g = np.arange(gp)[None, :, None, None]
    j = np.arange(2)[None, None, :, None]
    b = np.arange(4)[None, None, None, :]
    off = (oracle.word_offset2(k, rows, g, j) + b).reshape(-1)
    assert np.array_equal(np.sort(off), np.arange(L["code_plane_bytes"]))


def test_pack_round_trip_and_padding():
    rng = np.random.default_rng(1)
    n, k = 37, 160
    codes = rng.integers(0, 4, (n, k), dtype=np.uint8)
    scales = rng.integers(100, 140, (n, k // 32), dtype=np.uint8)
    cp, sp = oracle.pack2(codes, scales)
    c2, s2 = oracle.unpack2(cp, sp, n, k)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    # bytes of padding rows and groups stay zero
    owned = np.zeros(cp.size, bool)
    for r in range(n):
        for g in range(k // 32):
            for j in range(2):
                o = int(oracle.word_offset2(k, r, g, j))
                owned[o:o + 4] = True
    assert not cp[~owned].any()


def _torch_w2(codes, scales, cb4):
    cbv = torch.from_numpy(cb4).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    w = cbv[np.arange(codes.shape[0])[:, None], codes.astype(np.int64) & 3]
    return w * np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=1)


def test_linear2_against_torch_decode():
    rng = np.random.default_rng(2)
    n, k, m = 50, 320, 3
    codes = rng.integers(0, 4, (n, k), dtype=np.uint8)
    scales = rng.integers(117, 124, (n, k // 32), dtype=np.uint8)
    cb4 = torch.randn(n, 4).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    x = torch.randn(m, k).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    cp, sp = oracle.pack2(codes, scales)
    y, bound = oracle.linear2(cp, sp, cb4, n, k, xb)
    w = _torch_w2(codes, scales, cb4)
    xr = x.to(torch.float64).numpy()
    assert np.allclose(y, xr @ w.T, rtol=0, atol=1e-12)
    assert np.allclose(bound, np.abs(xr) @ np.abs(w).T, rtol=0, atol=1e-12)


def test_linear2_worked_value_and_closed_forms():
    val = float(_rows("value")[0])
    k = 32
    cb4 = np.array([[0x38, 0x40, 0xB8, 0x30]], dtype=np.uint8)
    codes = (np.arange(k) % 4).astype(np.uint8)[None, :]
    scales = np.array([[126]], dtype=np.uint8)
    x = np.full((1, k), 0x3F80, dtype=np.uint16)
    cp, sp = oracle.pack2(codes, scales)
    y, _ = oracle.linear2(cp, sp, cb4, 1, k, x)
    assert y[0, 0] == val
    # one-hot codebook: the product counts the activations that hit that code
    for hot in range(4):
        cbh = np.zeros((1, 4), dtype=np.uint8)
        cbh[0, hot] = 0x38
        y, _ = oracle.linear2(cp, sp, cbh, 1, k, x)
        assert y[0, 0] == 0.5 * (k // 4)


def test_linear2_exact_fraction_brute_force():
    rng = np.random.default_rng(3)
    n, k = 3, 64
    codes = rng.integers(0, 4, (n, k), dtype=np.uint8)
    scales = rng.integers(120, 130, (n, k // 32), dtype=np.uint8)
    cb4 = rng.integers(0, 0x7E, (n, 4), dtype=np.uint8)
    x = torch.randn(2, k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    cp, sp = oracle.pack2(codes, scales)
    y, _ = oracle.linear2(cp, sp, cb4, n, k, x)

    def e4m3(b):
        s = -1 if b & 0x80 else 1
        e, mant = (b >> 3) & 15, b & 7
        return s * (Fraction(mant, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(mant, 8)) * Fraction(2) ** (e - 7))

    def bf16(bits):
        return Fraction(float(np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0]))

    for mi in range(2):
        for r in range(n):
            exact = sum(bf16(x[mi, kk]) * e4m3(int(cb4[r, codes[r, kk]])) * Fraction(2) ** (int(scales[r, kk // 32]) - 127)
                        for kk in range(k))
            assert abs(Fraction(y[mi, r]) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 80)


def test_shortlist_ties_and_brute_force():
    want = [int(v) for v in _rows("shortlist")[0].split()]
    assert oracle.shortlist(np.array([[1.0, 3.0, 3.0, 2.0, 3.0]]), 3)[0].tolist() == want
    rng = np.random.default_rng(4)
    s = rng.integers(0, 6, (5, 40)).astype(np.float32)     # many ties
    got = oracle.shortlist(s, 16)
    for i in range(5):
        order = sorted(range(40), key=lambda r: (-s[i, r], r))
        assert got[i].tolist() == order[:16]
    d = rng.standard_normal((3, 1000)).astype(np.float32)  # distinct scores
    assert np.array_equal(oracle.shortlist(d, 16), torch.topk(torch.from_numpy(d), 16).indices.numpy())


def test_mxfp8_and_rescore_against_torch():
    rng = np.random.default_rng(5)
    n, k, m = 40, 256, 2
    e8 = torch.randn(n, k).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    s8 = rng.integers(120, 130, (n, k // 32), dtype=np.uint8)
    w = torch.from_numpy(e8).view(torch.float8_e4m3fn).to(torch.float64).numpy() * \
        np.repeat(2.0 ** (s8.astype(np.float64) - 127), 32, axis=1)
    assert np.array_equal(oracle.mxfp8_dequantize(e8, s8), w)
    x = torch.randn(m, k).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    ids = np.array([[3, 9, 0, 39], [5, 5, 17, 2]], dtype=np.int32)
    y, bound = oracle.rescore(e8, s8, xb, ids)
    xr = x.to(torch.float64).numpy()
    for i in range(m):
        assert np.allclose(y[i], w[ids[i]] @ xr[i], rtol=0, atol=1e-12)
        assert np.allclose(bound[i], np.abs(w[ids[i]]) @ np.abs(xr[i]), rtol=0, atol=1e-12)


def test_decide_brute_force():
    ids = np.array([[7, 3, 9, 1], [4, 2, 8, 6]], dtype=np.int32)
    sc = np.array([[0.5, 2.0, 2.0, -1.0], [1.0, 1.0, 1.0, 1.0]])
    assert oracle.decide(ids, sc).tolist() == [3, 2]     # equal scores: the lower row wins
