"""CPU oracle for the two-bit draft head: candidates picked on a 2-bit copy, the choice made on FP8 weights.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the GPU path
and imports nothing from it; numbers are decoded with the (pinned) helpers of
the 3-bit oracle next to it.

What it computes (Hibana: Fast Agentic Inference on Unified-Memory Devices --
"Model surgery", subsection "Two-bit draft head"): the drafter's vocabulary
projection is evaluated on a 2-bit copy to pick a short list of candidate
tokens, and only those candidates are evaluated again with the FP8 weights,
which make the choice:

    s2[m][n] = sum_k x[m][k] * w2[n][k]                 (all n, 2-bit head)
    L[m]     = the S rows with the largest s2[m][.]     (S = 16 on the page)
    s8[m][j] = sum_k x[m][k] * w8[L[m][j]][k]           (FP8 head, S rows only)
    best[m]  = the row of L[m] with the largest s8

Readings taken where the page is silent (each also listed in the design notes):
  * the 2-bit copy mirrors the 3-bit format: a 4-entry E4M3FN codebook per
    row, 2-bit indices, one E8M0 scale per group of 32, i.e. 2 + 8/32 =
    2.25 bits per weight;
        w2[n][k] = E4M3FN(cb4[n][code]) * 2^(scale[n][k // 32] - 127)
  * the 64 code bits of a group sit in two words in a byte-lane order (see
    pack_group2) and the words and scale bytes are placed in tiles of 16 rows
    and steps of 16 groups exactly like the 3-bit planes, with two words per
    group instead of three (see word_offset2; the scale plane is identical);
  * "FP8" for the rescoring head is OCP MXFP8: E4M3FN elements with one E8M0
    scale per 32 consecutive elements of a row, stored row-major,
        w8[n][k] = E4M3FN(e8[n][k]) * 2^(s8[n][k // 32] - 127);
  * ranking: larger score first, equal scores to the lower row index (so the
    list and the decision are unique);
  * activations bf16, scores fp32 (oracle: fp64).

Parity status per function (pins in tests/test_oracle_head.py):
  layout2          pinned: payload = n*k*9/32 (2.25 bits/weight closed form)
  pack_group2      pinned: hand-derived worked example, brute-force round trip
  word_offset2     pinned: hand-derived offsets; every plane byte owned once
  pack2/unpack2    pinned: round trip, padding zero
  linear2          pinned: torch fp64 matmul of torch-decoded weights, closed
                   forms, exact Fraction brute force on tiny K
  shortlist        pinned: brute-force sort with ties; torch.topk on distinct scores
  mxfp8_dequantize pinned: torch float8_e4m3fn decode times 2^(s-127)
  rescore          pinned: torch fp64 matmul of the gathered rows
  decide           pinned: brute force over the list, ties to the lower row
"""
from __future__ import annotations

import numpy as np

from .q3_oracle import E4M3FN_TABLE, GROUP, QUAD, STEP_GROUPS, TILE_ROWS, bf16_decode, e8m0_decode, scale_offset

CODEBOOK2_SIZE = 4          # 2-bit indices
CODE2_BYTES_PER_GROUP = 8   # 64 code bits
SHORTLIST = 16              # rows kept by the 2-bit pass on the page


# ------------------------------------------------------------------ layout

def layout2(n: int, k: int) -> dict:
    """Sizes of the 2-bit planes of an n x k head.

    Same tiling as the 3-bit planes (rows padded to 16, groups to a multiple
    of 4), 8 code bytes per group instead of 12.  Codebook: 4 bytes per row.
    Payload counts only real codes and scales: k/32 * 9 bytes per row =
    n*k*9/32 bytes, i.e. 2.25 bits per weight.
    """
    if n < 0 or k <= 0 or k % GROUP:
        raise ValueError("k must be a positive multiple of 32")
    groups = k // GROUP
    padded = -(-groups // QUAD) * QUAD
    tiles = -(-n // TILE_ROWS)
    code_tile = TILE_ROWS * CODE2_BYTES_PER_GROUP * padded
    scale_tile = TILE_ROWS * padded
    return dict(n=n, k=k, groups=groups, padded_groups=padded, tiles=tiles,
                code_tile_bytes=code_tile, scale_tile_bytes=scale_tile,
                code_plane_bytes=tiles * code_tile, scale_plane_bytes=tiles * scale_tile,
                codebook_bytes=n * CODEBOOK2_SIZE,
                payload_bytes=n * groups * (CODE2_BYTES_PER_GROUP + 1))


# --------------------------------------------------------------- bit layout

def pack_group2(c) -> tuple:
    """32 codes (0..3, K order) -> two little-endian uint32 words.

    Byte b (0..3) of word j (0..1) holds code 16j+4q+b in bits 2q..2q+1
    (q = 0..3), so shifting a word right by 2q and masking 0x03 per byte
    yields four codes in K order.
    """
    c = [int(v) & 3 for v in c]
    assert len(c) == GROUP
    words = []
    for j in range(2):
        w = 0
        for b in range(4):
            byte = 0
            for q in range(4):
                byte |= c[16 * j + 4 * q + b] << (2 * q)
            w |= byte << (8 * b)
        words.append(w)
    return tuple(words)


def unpack_group2(words) -> list:
    """Inverse of pack_group2: two uint32 words -> 32 codes in K order."""
    c = [0] * GROUP
    for j in range(2):
        for b in range(4):
            byte = (int(words[j]) >> (8 * b)) & 0xFF
            for q in range(4):
                c[16 * j + 4 * q + b] = (byte >> (2 * q)) & 3
    return c


def _pack_bytes2(c):
    """Vectorised pack_group2: codes uint8 [..., 32] -> bytes uint8 [..., 8]
    (byte 4j+b of the group = byte b of word j)."""
    c = c.astype(np.uint8) & 3
    out = np.zeros(c.shape[:-1] + (8,), dtype=np.uint8)
    for j in range(2):
        for b in range(4):
            for q in range(4):
                out[..., 4 * j + b] |= c[..., 16 * j + 4 * q + b] << (2 * q)
    return out


def _unpack_bytes2(by):
    """Vectorised inverse: bytes uint8 [..., 8] -> codes uint8 [..., 32]."""
    c = np.empty(by.shape[:-1] + (32,), dtype=np.uint8)
    for j in range(2):
        for b in range(4):
            for q in range(4):
                c[..., 16 * j + 4 * q + b] = (by[..., 4 * j + b] >> (2 * q)) & 3
    return c


def word_offset2(k: int, r, g, j):
    """Code-plane byte offset of word j (0..1) of group g of row r.

    Tile T = r // 16 starts at T * 128 * Gp; step s = g // 16 starts 2048 * s
    bytes into it and holds 2 * 4q pieces of 16 bytes (q = quads of groups in
    the step); piece 16*(q*j + kb) + i is word j of quad kb of the tile's row
    i = r % 16, and 4-byte word t inside it belongs to group 16s+4kb+t.
    """
    gp = layout2(1, k)["padded_groups"]
    r = np.asarray(r, dtype=np.int64)
    g = np.asarray(g, dtype=np.int64)
    T, i = np.divmod(r, TILE_ROWS)
    s, u = np.divmod(g, STEP_GROUPS)
    kb, t = np.divmod(u, QUAD)
    q = np.minimum(STEP_GROUPS, gp - STEP_GROUPS * s) // QUAD
    return (T * TILE_ROWS * CODE2_BYTES_PER_GROUP * gp + 2048 * s
            + 16 * (16 * (q * np.asarray(j) + kb) + i) + 4 * t)


def _code_index2(k: int, rows) -> np.ndarray:
    G = k // GROUP
    r = np.asarray(rows, dtype=np.int64)[:, None, None, None]
    g = np.arange(G)[None, :, None, None]
    j = np.arange(2)[None, None, :, None]
    b = np.arange(4)[None, None, None, :]
    return (word_offset2(k, r, g, j) + b).reshape(len(rows), G, 8)


def _scale_index(k: int, rows) -> np.ndarray:
    G = k // GROUP
    return scale_offset(k, np.asarray(rows, dtype=np.int64)[:, None], np.arange(G)[None, :])


def pack2(codes: np.ndarray, scales: np.ndarray, block: int = 1024):
    """codes uint8 [n][k] (bits 0..1 used), scales uint8 [n][k/32] ->
    (code_plane, scale_plane) uint8, padding bytes zero."""
    n, k = codes.shape
    L = layout2(n, k)
    G = L["groups"]
    cp = np.zeros(L["code_plane_bytes"], dtype=np.uint8)
    sp = np.zeros(L["scale_plane_bytes"], dtype=np.uint8)
    for r0 in range(0, n, block):
        rows = np.arange(r0, min(n, r0 + block))
        cp[_code_index2(k, rows).reshape(-1)] = _pack_bytes2(codes[rows].reshape(len(rows), G, 32)).reshape(-1)
        sp[_scale_index(k, rows).reshape(-1)] = scales[rows].reshape(-1)
    return cp, sp


def unpack2(code_plane, scale_plane, n: int, k: int, rows=None):
    """Planes of an n x k 2-bit head -> (codes uint8 [len(rows)][k], scales uint8 [len(rows)][k/32])."""
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    by = np.asarray(code_plane)[_code_index2(k, rows)]
    return _unpack_bytes2(by).reshape(len(rows), k), np.asarray(scale_plane)[_scale_index(k, rows)]


# ---------------------------------------------------------------- products

def dequantize2(codes, scales, codebook4) -> np.ndarray:
    """w2[n][k] = E4M3FN(codebook4[n][codes & 3]) * 2^(scales[n][k/32] - 127), float64."""
    n, k = codes.shape
    cbv = E4M3FN_TABLE[np.asarray(codebook4).astype(np.int64)]     # [n][4]
    w = cbv[np.arange(n)[:, None], (codes & 3).astype(np.int64)]
    return w * np.repeat(e8m0_decode(scales), GROUP, axis=1)


def linear2(code_plane, scale_plane, codebook4, n, k, x_bits, rows=None, block=2048):
    """s2[m][r] = sum_k x[m][k] w2[r][k] and its bound sum_k |x w2| in fp64,
    weights read back from the planes with this module's own unpacking."""
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    x = bf16_decode(x_bits)
    xa = np.abs(x)
    y = np.empty((x.shape[0], rows.size))
    bound = np.empty_like(y)
    for s in range(0, rows.size, block):
        r = rows[s:s + block]
        codes, scales = unpack2(code_plane, scale_plane, n, k, rows=r)
        w = dequantize2(codes, scales, np.asarray(codebook4)[r])
        y[:, s:s + r.size] = x @ w.T
        bound[:, s:s + r.size] = xa @ np.abs(w).T
    return y, bound


def shortlist(scores, size: int = SHORTLIST) -> np.ndarray:
    """Rows of the `size` largest scores of each query, largest first; equal
    scores go to the lower row index.  int32 [m][size]."""
    scores = np.asarray(scores)
    m, n = scores.shape
    out = np.empty((m, size), dtype=np.int32)
    idx = np.arange(n)
    for i in range(m):
        order = np.lexsort((idx, -scores[i].astype(np.float64)))
        out[i] = order[:size]
    return out


def mxfp8_dequantize(e8, s8) -> np.ndarray:
    """w8[n][k] = E4M3FN(e8[n][k]) * 2^(s8[n][k/32] - 127), float64."""
    e8 = np.asarray(e8)
    return E4M3FN_TABLE[e8.astype(np.int64)] * np.repeat(e8m0_decode(s8), GROUP, axis=1)


def rescore(e8, s8, x_bits, ids):
    """s8[m][j] = sum_k x[m][k] w8[ids[m][j]][k] and its bound, fp64."""
    x = bf16_decode(x_bits)
    ids = np.asarray(ids)
    y = np.empty(ids.shape)
    bound = np.empty(ids.shape)
    for i in range(ids.shape[0]):
        w = mxfp8_dequantize(np.asarray(e8)[ids[i]], np.asarray(s8)[ids[i]])
        y[i] = w @ x[i]
        bound[i] = np.abs(w) @ np.abs(x[i])
    return y, bound


def decide(ids, scores8) -> np.ndarray:
    """The listed row with the largest FP8 score per query (equal scores: lower row)."""
    ids = np.asarray(ids)
    best = np.empty(ids.shape[0], dtype=np.int32)
    for i in range(ids.shape[0]):
        j = min(range(ids.shape[1]), key=lambda j: (-float(scores8[i][j]), int(ids[i][j])))
        best[i] = ids[i][j]
    return best
