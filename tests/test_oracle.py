"""Pins of the CPU oracle against facts that do not come from the oracle itself:
the page's 3.25 bits/weight, the OFP8/MX number definitions, library decoders
(torch.float8_e4m3fn, torch.bfloat16, torch float64 matmul), a hand-derived
worked example of the bit layout, closed forms and exact rational brute force.
The last block plants mistakes in the oracle and checks that a pin catches each."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import golden_kv, read_golden

CONFIG_SHAPES = [(1024, 1024), (4096, 4096), (1536, 2048), (2048, 768), (28672, 8192), (151936, 4096)]


# ------------------------------------------------------------------ numbers

def e4m3_table_matches_torch(table):
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    return (np.array_equal(np.isnan(table), nan) and np.array_equal(table[~nan], ref[~nan])
            and np.array_equal(np.signbit(table[~nan]), np.signbit(ref[~nan])))


def test_e4m3fn_all_bytes_match_torch():
    assert e4m3_table_matches_torch(oracle.E4M3FN_TABLE)


def test_e4m3fn_spec_points():
    for row in read_golden("e4m3fn_points.txt"):
        b, v = row.split()
        got = oracle.e4m3fn_decode(int(b, 16))
        if v == "nan":
            assert math.isnan(got)
        else:
            assert got == float(v) and math.copysign(1, got) == math.copysign(1, float(v)), (b, got)


def test_e8m0_spec_points():
    for row in read_golden("e8m0_points.txt"):
        b, e = row.split()
        got = float(oracle.e8m0_decode(int(b, 16)))
        if e == "nan":
            assert math.isnan(got)
        else:
            assert got == math.ldexp(1.0, int(e))


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    bits = np.concatenate([rng.integers(0, 1 << 16, 4096, dtype=np.uint16),
                           np.array([0x0000, 0x8000, 0x0001, 0x7F7F, 0x3F80, 0xBF80, 0x7F80], dtype=np.uint16)])
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_decode(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ------------------------------------------------------------------- format

def test_payload_is_3p25_bits_per_weight():
    kv = golden_kv("bits_per_weight.txt")
    bpw = float(kv["bits_per_weight"])
    assert int(kv["code_bits"]) + int(kv["scale_bits"]) / int(kv["group"]) == bpw
    for n, k in CONFIG_SHAPES:
        L = oracle.layout(n, k)
        assert L["payload_bytes"] * 8 == n * k * bpw
        assert L["payload_bytes"] == n * k * 13 // 32
        # With n a multiple of 16 and k of 128 the planes hold exactly the payload.
        if n % 16 == 0 and k % 128 == 0:
            assert L["code_plane_bytes"] + L["scale_plane_bytes"] == L["payload_bytes"]
    assert oracle.layout(1024, 1024)["payload_bytes"] == 425984
    assert oracle.layout(4096, 4096)["payload_bytes"] == 6815744
    assert oracle.layout(28672, 8192)["payload_bytes"] == 95420416
    assert oracle.layout(151936, 4096)["payload_bytes"] == 252821504


def test_worked_example():
    kv = golden_kv("format_worked_example.txt")
    codes = [int(v) for v in kv["codes"].split(",")]
    words = tuple(int(v, 16) for v in kv["words"].split(","))
    assert oracle.pack_group(codes) == words
    assert oracle.unpack_group(words) == codes
    cp, sp = oracle.pack(np.array(codes, dtype=np.uint8)[None, :], np.array([[127]], dtype=np.uint8))
    # k = 32, one row: the tile's single step holds one quad (q = 1), so word j
    # of row 0's group is the first word of piece 16*j, at byte 256*j.
    assert cp.size == 16 * 12 * 4 and sp.size == 16 * 4
    for j, w in enumerate(words):
        assert cp[256 * j:256 * j + 4].tobytes() == w.to_bytes(4, "little")
    assert not np.delete(cp, [b for j in range(3) for b in range(256 * j, 256 * j + 4)]).any()
    assert sp[0] == 127 and not sp[1:].any()


def test_word_placement_worked_examples():
    for row in read_golden("word_placement.txt"):
        plane, k, r, g, j, byte = row.split()
        k, r, g, byte = int(k), int(r), int(g), int(byte)
        if plane == "code":
            assert int(oracle.word_offset(k, r, g, int(j))) == byte, (k, r, g, j)
        else:
            assert int(oracle.scale_offset(k, r, g)) == byte, (k, r, g)


@pytest.mark.parametrize("n,k", [(1, 32), (16, 96), (17, 128), (3, 160), (33, 640), (16, 768), (5, 1024),
                                 (2, 4096), (1, 8224)])
def test_placement_covers_each_plane_byte_once(n, k):
    """Over all rows of the padded tiles and all padded groups, every code-plane
    byte belongs to exactly one (row, group, word, byte) and every scale-plane
    byte to exactly one (row, group)."""
    L = oracle.layout(n, k)
    rows = np.arange(16 * L["tiles"])[:, None, None, None]
    g = np.arange(L["padded_groups"])[None, :, None, None]
    j = np.arange(3)[None, None, :, None]
    b = np.arange(4)[None, None, None, :]
    cover = np.zeros(L["code_plane_bytes"], dtype=np.int64)
    np.add.at(cover, (oracle.word_offset(k, rows, g, j) + b).reshape(-1), 1)
    assert np.all(cover == 1)
    scover = np.zeros(L["scale_plane_bytes"], dtype=np.int64)
    np.add.at(scover, oracle.scale_offset(k, rows[..., 0, 0], g[..., 0, 0]).reshape(-1), 1)
    assert np.all(scover == 1)


def test_step_words_are_contiguous_runs():
    """Word j of one quad index of a full step is a contiguous 256-byte run over
    the tile's 16 rows (16 bytes per row), and the scales of a full step are one
    256-byte run: a 64-lane load of the step reads 1 KB or 256 B contiguous."""
    k = 1024
    for j in range(3):
        offs = sorted(int(oracle.word_offset(k, i, 16 + 4 * kb, j)) for kb in range(4) for i in range(16))
        assert offs == list(range(offs[0], offs[0] + 64 * 16, 16)) and offs[0] == 3072 + 1024 * j
    soffs = sorted(int(oracle.scale_offset(k, i, 16 + 4 * kb)) for kb in range(4) for i in range(16))
    assert soffs == list(range(256, 512, 4))


def test_each_code_position_owns_three_distinct_bits():
    """Bijectivity: the 32 positions x 3 bits partition the 96 bits of a group."""
    seen = 0
    for pos in range(32):
        for v in range(8):
            c = [0] * 32
            c[pos] = v
            w = oracle.pack_group(c)
            big = w[0] | (w[1] << 32) | (w[2] << 64)
            assert bin(big).count("1") == bin(v).count("1")
            assert oracle.unpack_group(w) == c
        c = [0] * 32
        c[pos] = 7
        w = oracle.pack_group(c)
        big = w[0] | (w[1] << 32) | (w[2] << 64)
        assert big & seen == 0
        seen |= big
    assert seen == (1 << 96) - 1


def test_group_roundtrip_random_and_vectorised_agree():
    rng = np.random.default_rng(2)
    c = rng.integers(0, 8, size=(2000, 32), dtype=np.uint8)
    by = oracle.q3_oracle._pack_bytes(c)
    for i in range(0, 2000, 97):
        words = oracle.pack_group(c[i])
        assert by[i].tobytes() == b"".join(w.to_bytes(4, "little") for w in words)
        assert oracle.unpack_group(words) == list(c[i])
    assert np.array_equal(oracle.q3_oracle._unpack_bytes(by), c)


@pytest.mark.parametrize("n,k", [(3, 32), (5, 96), (7, 128), (4, 160), (9, 768), (2, 4096), (18, 640)])
def test_plane_roundtrip_padding_and_masking(n, k):
    rng = np.random.default_rng(n * 1000 + k)
    codes = rng.integers(0, 256, size=(n, k), dtype=np.uint8)     # high bits must be ignored
    scales = rng.integers(0, 255, size=(n, k // 32), dtype=np.uint8)
    cp, sp = oracle.pack(codes, scales)
    L = oracle.layout(n, k)
    assert cp.shape == (L["code_plane_bytes"],) and sp.shape == (L["scale_plane_bytes"],)
    G = k // 32
    # Bytes of padding rows and padding groups are zero.
    rows = np.arange(16 * L["tiles"])
    real = (rows[:, None] < n) & (np.arange(L["padded_groups"])[None, :] < G)
    g = np.arange(L["padded_groups"])
    woff = oracle.word_offset(k, rows[:, None, None], g[None, :, None], np.arange(3)[None, None, :])
    pad = (woff[~real][..., None] + np.arange(4)).reshape(-1)
    assert not cp[pad].any()
    assert not sp[oracle.scale_offset(k, rows[:, None], g[None, :])[~real]].any()
    c2, s2 = oracle.unpack(cp, sp, n, k)
    assert np.array_equal(c2, codes & 7) and np.array_equal(s2, scales)
    sub = np.array([n - 1, 0])
    c3, s3 = oracle.unpack(cp, sp, n, k, rows=sub)
    assert np.array_equal(c3, codes[sub] & 7) and np.array_equal(s3, scales[sub])


# ------------------------------------------------------------------ products

def torch_dequant(layer):
    """Independent dequantisation with library decoders: torch's E4M3FN cast and torch.ldexp."""
    cb = torch.from_numpy(layer.codebook).view(torch.float8_e4m3fn).to(torch.float64)
    codes = torch.from_numpy(layer.codes.astype(np.int64) & 7)
    w = torch.gather(cb, 1, codes)
    e = torch.from_numpy(layer.scales.astype(np.int64) - 127).repeat_interleave(32, dim=1)
    return torch.ldexp(w, e.to(torch.float64))


def torch_x(x_bits):
    return torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)


def oracle_y(layer, x_bits, rows=None):
    cp, sp = oracle.pack(layer.codes, layer.scales)
    return oracle.linear(cp, sp, layer.codebook, layer.n, layer.k, x_bits, rows=rows)


@pytest.mark.parametrize("n,k,m", [(64, 1024, 1), (33, 4096, 4), (20, 768, 8), (7, 96, 3), (16, 8192, 16)])
def test_linear_matches_torch_fp64_matmul(n, k, m):
    layer, x = synth.make_linear(n, k, m, seed=n + k + m)
    y, bound = oracle_y(layer, x)
    ref = (torch_x(x) @ torch_dequant(layer).T).numpy()
    assert np.all(np.abs(y - ref) <= 1e-12 * bound)
    refb = (torch_x(x).abs() @ torch_dequant(layer).abs().T).numpy()
    assert np.allclose(bound, refb, rtol=1e-12, atol=0)


def test_linear_rows_subset_matches_full():
    layer, x = synth.make_linear(50, 256, 2, seed=5)
    y, b = oracle_y(layer, x)
    rows = [49, 3, 17]
    ys, bs = oracle_y(layer, x, rows=rows)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(bs, b[:, rows])


def _xvals(x_bits):
    return [[float(v) for v in row] for row in torch_x(x_bits).numpy()]


def test_closed_form_one_hot_codebook():
    """cb[j] = 1.0, others 0: y = sum_g 2^e_g * sum_{k in g, c_k = j} x_k."""
    layer, x = synth.make_linear(6, 128, 3, seed=11)
    for j in range(8):
        layer.codebook[:] = 0x00
        layer.codebook[:, j] = 0x38
        y, _ = oracle_y(layer, x)
        xv = _xvals(x)
        for m in range(3):
            for n in range(6):
                ref = 0.0
                for g in range(4):
                    part = sum(xv[m][k] for k in range(32 * g, 32 * g + 32) if layer.codes[n, k] == j)
                    ref += math.ldexp(part, int(layer.scales[n, g]) - 127)
                assert abs(y[m, n] - ref) <= 1e-12 * (1 + abs(ref))


def test_closed_form_constant_codes_and_single_group():
    layer, x = synth.make_linear(5, 32, 2, seed=12)   # K = 32: one group, one scale per row
    for j in range(8):
        layer.codes[:] = j
        y, _ = oracle_y(layer, x)
        xv = _xvals(x)
        for m in range(2):
            for n in range(5):
                cbj = float(torch.tensor([int(layer.codebook[n, j])], dtype=torch.uint8).view(torch.float8_e4m3fn).double())
                ref = cbj * math.ldexp(sum(xv[m]), int(layer.scales[n, 0]) - 127)
                assert abs(y[m, n] - ref) <= 1e-13 * (1 + abs(ref))


@pytest.mark.parametrize("k", [32, 64, 96])
def test_exact_rational_bruteforce(k):
    layer, x = synth.make_linear(4, k, 4, seed=k)
    layer.codebook[0, 3] = 0x80   # -0
    layer.codebook[1, :] = 0x38   # repeated entries
    layer.scales[2, 0] = 140      # spread of scales
    y, bound = oracle_y(layer, x)
    cbv = torch.from_numpy(layer.codebook).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    xv = _xvals(x)
    for m in range(4):
        for n in range(4):
            exact = Fraction(0)
            for kk in range(k):
                w = Fraction(float(cbv[n, layer.codes[n, kk]])) * Fraction(2) ** (int(layer.scales[n, kk // 32]) - 127)
                exact += Fraction(xv[m][kk]) * w
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(2) ** -50 * Fraction(bound[m, n])


def test_fp32_accumulation_meets_tolerance_by_construction():
    """Products x*w are exact in fp32 (8 x 4 significant bits); recursive fp32
    summation then errs by at most gamma_K * sum|x w|, gamma_K = K u/(1-K u),
    u = 2^-24, which is below 1e-3 for every K used (K <= 8192)."""
    u = 2.0 ** -24
    for k in (768, 1024, 2048, 4096, 8192):
        assert k * u / (1 - k * u) < 1e-3
    layer, x = synth.make_linear(8, 8192, 1, seed=3)
    y, bound = oracle_y(layer, x)
    w = torch_dequant(layer).numpy().astype(np.float32)
    xf = torch_x(x).numpy().astype(np.float32)[0]
    prods = (w * xf[None, :]).astype(np.float32)
    assert np.array_equal(prods.astype(np.float64), w.astype(np.float64) * xf.astype(np.float64)[None, :])
    for order in (np.arange(8192), np.random.default_rng(0).permutation(8192)):
        acc = np.zeros(8, dtype=np.float32)
        for kk in order:
            acc = (acc + prods[:, kk]).astype(np.float32)
        ok, ratio = oracle.within_tolerance(acc[None, :], y, bound)
        assert ok and ratio < 2.5e-4


def test_within_tolerance_rule():
    y_ref = np.array([[1.0, 0.0]])
    bound = np.array([[10.0, 0.0]])
    assert oracle.within_tolerance(np.array([[1.0 + 0.0099, 0.0]]), y_ref, bound)[0]
    assert not oracle.within_tolerance(np.array([[1.0 + 0.011, 0.0]]), y_ref, bound)[0]
    assert not oracle.within_tolerance(np.array([[1.0, 1e-30]]), y_ref, bound)[0]


# ---------------------------------------------------------------------- MoE

def test_topk_route_bruteforce_and_ties():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((6, 10)).astype(np.float32)
    ids = oracle.topk_route(logits, 3)
    for t in range(6):
        best = max(itertools.combinations(range(10), 3), key=lambda s: sum(float(logits[t, e]) for e in s))
        assert set(ids[t]) == set(best)
        assert list(logits[t, ids[t]]) == sorted(logits[t, ids[t]], reverse=True)
    tv, ti = torch.topk(torch.from_numpy(logits), 3, dim=1)
    assert np.array_equal(ti.numpy(), ids)
    tie = np.zeros((1, 8), dtype=np.float32)
    tie[0, [6, 2, 5]] = 1.0
    assert list(oracle.topk_route(tie, 4)[0]) == [2, 5, 6, 0]


def test_union_expected_size_config2():
    """8 tokens x top-8 of 64: a given expert is missed by one token w.p. 7/8,
    so E|U| = 64 (1 - (7/8)^8) ~= 42.0; check the seeded union is plausible and
    the union bytes are |U| * (gate/up + down payload)."""
    assert abs(64 * (1 - (7 / 8) ** 8) - 42.0) < 0.05
    moe = synth.make_moe(num_experts=64, k_gu=64, n_gu=8, k_dn=32, n_dn=8)
    ids = oracle.topk_route(moe.logits, 8)
    u = oracle.expert_union(ids)
    assert 20 <= u.size <= 64 and np.all(np.diff(u) > 0)
    per_expert = oracle.layout(1536, 2048)["payload_bytes"] + oracle.layout(2048, 768)["payload_bytes"]
    assert per_expert == 1916928


def test_grouped_equals_per_pair_dense():
    moe = synth.make_moe(num_experts=6, k_gu=64, n_gu=24, k_dn=96, n_dn=16, tokens=3, topk=2, seed=9)
    ids = oracle.topk_route(moe.logits, 2)
    planes_gu = [(*oracle.pack(L.codes, L.scales), L.codebook, L.n, L.k) for L in moe.experts_gu]
    planes_dn = [(*oracle.pack(L.codes, L.scales), L.codebook, L.n, L.k) for L in moe.experts_dn]
    y, b = oracle.grouped_linear(planes_gu, ids, moe.x, False)
    yd, bd = oracle.grouped_linear(planes_dn, ids, moe.x_dn[:, :2], True)
    for t in range(3):
        for j in range(2):
            e = ids[t, j]
            ref = (torch_x(moe.x[t:t + 1]) @ torch_dequant(moe.experts_gu[e]).T).numpy()[0]
            assert np.allclose(y[t, j], ref, rtol=0, atol=1e-12 * b[t, j].max())
            refd = (torch_x(moe.x_dn[t, j][None]) @ torch_dequant(moe.experts_dn[e]).T).numpy()[0]
            assert np.allclose(yd[t, j], refd, rtol=0, atol=1e-12 * bd[t, j].max())


# ------------------------------------------------------- planted mistakes

def test_planted_fnuz_bias_is_caught():
    """E4M3FNUZ (bias 8) instead of E4M3FN must fail the torch comparison."""
    def fnuz(b):
        v = oracle.e4m3fn_decode(b)
        return v / 2 if not math.isnan(v) else v
    assert not e4m3_table_matches_torch(np.array([fnuz(b) for b in range(256)]))


def test_planted_spill_swap_is_caught():
    kv = golden_kv("format_worked_example.txt")
    codes = [int(v) for v in kv["codes"].split(",")]
    words = tuple(int(v, 16) for v in kv["words"].split(","))
    c = list(codes)
    c[24:28], c[28:32] = c[28:32], c[24:28]    # packer that swaps the two spilled quartets
    assert oracle.pack_group(c) != words


def test_planted_dropped_scale_and_transpose_are_caught(monkeypatch):
    layer, x = synth.make_linear(12, 256, 2, seed=21)
    ref = (torch_x(x) @ torch_dequant(layer).T).numpy()
    real = oracle.q3_oracle.dequantize

    def no_scale(codes, scales, codebook):
        return real(codes, np.full_like(scales, 127), codebook)
    monkeypatch.setattr(oracle.q3_oracle, "dequantize", no_scale)
    y, b = oracle_y(layer, x)
    assert not np.all(np.abs(y - ref) <= 1e-12 * b)

    def wrong_row(codes, scales, codebook):
        return real(codes, scales, codebook[::-1].copy())
    monkeypatch.setattr(oracle.q3_oracle, "dequantize", wrong_row)
    y, b = oracle_y(layer, x)
    assert not np.all(np.abs(y - ref) <= 1e-12 * b)
