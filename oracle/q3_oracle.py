"""CPU oracle for the 3-bit FP8-codebook decode linear layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the GPU path
(no kernels, headers, tables or helpers) and imports nothing from it; it is a
plain, slow, obviously-correct restatement of what the layer computes, in
float64 with numpy.

What the layer computes (Hibana: Fast Agentic Inference on Unified-Memory
Devices -- "Model surgery", subsection "Three-bit weights"): every group of 32
consecutive weights of a row is stored as 3-bit indices into an 8-entry FP8
codebook, plus one 8-bit scale per group, 3 + 8/32 = 3.25 bits per weight.
A decode step multiplies the dequantised matrix by a handful of token
activations:

    w[n][k] = E4M3FN(codebook[n][code[n][k]]) * 2^(scale[n][k // 32] - 127)
    y[m][n] = sum_k x[m][k] * w[n][k]

Readings taken where the page is silent (each also listed in the design notes):
  * one 8-entry codebook per output row (its 8 bytes are outside the 3.25
    bits/weight count, which only has codes and scales);
  * "FP8" is OCP E4M3FN (bias 7, max 448, NaN = 0x7F/0xFF, has -0);
  * the "8-bit scale" is an OCP-MX E8M0 power of two, value 2^(s-127);
  * the scale multiplies the codebook value;
  * activations are bf16, outputs fp32 (oracle: fp64);
  * the bit order of the 96 code bits of a group is this project's own
    "byte-lane" layout (see pack_group), and so is the placement of the
    words and scale bytes in the planes (tiles of 16 rows, steps of 16
    groups; see word_offset and scale_offset).
MoE verify rounds (same page, "Adaptive speculation" -- "Expert sharing"): a
round that checks several drafted tokens at once must read the weights of
each expert chosen by at least one of those tokens; the oracle routes each
token to its top-k experts by router logit (ties to the lower expert index)
and reports that union.

Parity status per function (what pins each one lives in tests/test_oracle.py):
  e4m3fn_decode   pinned: all 256 bytes vs torch.float8_e4m3fn, spec values
  e8m0_decode     pinned: spec values of the OCP MX E8M0 type
  bf16_decode     pinned: torch.bfloat16 for random and special bit patterns
  layout          pinned: payload = n*k*13/32 (3.25 bits/weight closed form)
  pack_group      pinned: hand-derived worked example, brute-force round trip
  word_offset,    pinned: hand-derived offsets, every plane byte owned by
  scale_offset            exactly one (row, group, word, byte) / (row, group)
  pack/unpack     pinned: round trip, worked examples, padding is zero
  linear          pinned: torch fp64 matmul of torch-decoded weights, closed
                  forms (one-hot codebook, constant codes, single group),
                  exact Fraction brute force on tiny K
  topk_route      pinned: brute-force ranking, torch.topk on distinct logits
  grouped_linear  pinned: equals per-(token, slot) dense linear calls
  moe_mlp         pinned: closed form on constant weights (silu of a known
                  sum, softmax of two logits), a torch float64 composition
                  from torch-decoded weights with F.silu and a renormalised
                  full softmax, and the bound's derivatives against autograd
  budget_route    pinned: brute force over expert subsets (largest total mass),
                  brute-force per-token ranking inside the set, budget = all
                  experts reduces to topk_route, and a hand-built instance
                  that reproduces every number of the page's toy figure

Fused expert MLP of a verify round (same page, "Expert sharing", the experts
the round reads).  Readings taken (the page gives no MLP detail): an expert's
gate/up matrix stacks the gate rows [0, I) over the up rows [I, 2I); the
hidden value is h = silu(g) * u with silu(z) = z / (1 + e^-z); each token's
output is the sum over its slots of p_s * (down_expert . h), where p is the
softmax of the token's routed logits (its top-k probabilities renormalised).
The allowance of a fused output is 1e-3 times its first-order error bound:
sum_s p_s sum_j |w_j| (|h_j| + |dh/dg_j| Bg_j + |dh/du_j| Bu_j), with Bg, Bu
the sums |x w| of the gate and up products (the layer's own allowance,
carried through the SwiGLU and the down product).

Expert budget (same page, "Adaptive speculation" -- "Expert sharing"): a verify
round gets a shared budget of experts; choices outside it are replaced by
choices inside it.  Reading taken (the policy is not spelled out): the round
keeps the `budget` experts with the largest total routing mass (sum over the
round's tokens of the softmax probability of the expert; equal mass: lower
index), and each token routes to its top-k experts inside that set by logit
(equal logits: lower index).
"""
from __future__ import annotations

import numpy as np

GROUP = 32                 # weights per group (one scale each)
CODEBOOK_SIZE = 8          # 3-bit indices
QUAD = 4                   # groups per 16-byte piece (one word of each)
CODE_BYTES_PER_GROUP = 12  # 96 code bits
TILE_ROWS = 16             # rows per tile
STEP_GROUPS = 16           # groups per step (512 weights of a row)
E8M0_BIAS = 127


# ----------------------------------------------------------------- numbers

def e4m3fn_decode(byte: int) -> float:
    """One OCP E4M3FN byte -> its value (float64).

    Sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.  Exponent 0
    is subnormal (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN (no
    infinities); everything else is (1 + m/8) * 2^(e-7).
    """
    byte = int(byte) & 0xFF
    sign = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3FN_TABLE = np.array([e4m3fn_decode(b) for b in range(256)], dtype=np.float64)


def e8m0_decode(s) -> np.ndarray:
    """E8M0 scale byte(s) -> 2^(s-127) in float64; 255 is NaN."""
    s = np.asarray(s, dtype=np.int64)
    out = np.ldexp(np.ones(s.shape, dtype=np.float64), (s - E8M0_BIAS).astype(np.int32))
    return np.where(s == 255, np.nan, out)


def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64.  bf16 is the top half of an
    IEEE binary32, so widening is exact: place the bits in the high half."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ layout

def layout(n: int, k: int) -> dict:
    """Sizes of the packed planes for an n x k matrix.

    Groups of a row are padded to Gp = 4*ceil(k/128) (padding groups are zero)
    and rows to a multiple of 16 (padding rows are zero).  Both planes are cut
    into tiles of 16 rows, stored one after the other; inside a tile the
    groups form steps of 16 (the last step of a row holds p = 4, 8, 12 or 16).
    A tile holds 16 * 12 * Gp code bytes and 16 * Gp scale bytes; where each
    word and scale byte sits is given by word_offset and scale_offset.
    Codebook: 8 bytes per row.  Payload counts only real codes and scales:
    k/32 * 13 bytes per row = n*k*13/32 bytes, i.e. 3.25 bits per weight.
    """
    if n < 0 or k <= 0 or k % GROUP:
        raise ValueError("k must be a positive multiple of 32")
    groups = k // GROUP
    padded = -(-groups // QUAD) * QUAD
    tiles = -(-n // TILE_ROWS)
    code_tile = TILE_ROWS * CODE_BYTES_PER_GROUP * padded
    scale_tile = TILE_ROWS * padded
    return dict(n=n, k=k, groups=groups, padded_groups=padded, tiles=tiles,
                code_tile_bytes=code_tile, scale_tile_bytes=scale_tile,
                code_plane_bytes=tiles * code_tile, scale_plane_bytes=tiles * scale_tile,
                codebook_bytes=n * CODEBOOK_SIZE,
                payload_bytes=n * groups * (CODE_BYTES_PER_GROUP + 1))


# --------------------------------------------------------------- bit layout

def pack_group(c) -> tuple:
    """32 codes (0..7, K order) -> three little-endian uint32 words.

    Byte b (0..3) of word j (0..2) holds
        bits 0..2: code 8j+b
        bits 3..5: code 8j+4+b
        bits 6..7: bits 2j..2j+1 of the six-bit value c[24+b] | c[28+b] << 3
    so masking a word with 0x07 per byte yields four codes in K order, and the
    last eight codes are spread two bits at a time over the top of all bytes.
    """
    c = [int(v) & 7 for v in c]
    assert len(c) == GROUP
    words = []
    for j in range(3):
        w = 0
        for b in range(4):
            spill = c[24 + b] | (c[28 + b] << 3)
            byte = c[8 * j + b] | (c[8 * j + 4 + b] << 3) | (((spill >> (2 * j)) & 3) << 6)
            w |= byte << (8 * b)
        words.append(w)
    return tuple(words)


def unpack_group(words) -> list:
    """Inverse of pack_group: three uint32 words -> 32 codes in K order."""
    c = [0] * GROUP
    spill = [0, 0, 0, 0]
    for j in range(3):
        for b in range(4):
            byte = (int(words[j]) >> (8 * b)) & 0xFF
            c[8 * j + b] = byte & 7
            c[8 * j + 4 + b] = (byte >> 3) & 7
            spill[b] |= ((byte >> 6) & 3) << (2 * j)
    for b in range(4):
        c[24 + b] = spill[b] & 7
        c[28 + b] = (spill[b] >> 3) & 7
    return c


def _pack_bytes(c):
    """Vectorised byte-lane packing: c uint8 [..., 32] -> bytes uint8 [..., 12]
    (byte 4j+b of the group = byte b of word j), same rule as pack_group."""
    c = c.astype(np.uint8) & 7
    out = np.empty(c.shape[:-1] + (12,), dtype=np.uint8)
    for b in range(4):
        spill = c[..., 24 + b] | (c[..., 28 + b] << 3)
        for j in range(3):
            out[..., 4 * j + b] = (c[..., 8 * j + b] | (c[..., 8 * j + 4 + b] << 3)
                                   | (((spill >> (2 * j)) & 3) << 6))
    return out


def _unpack_bytes(by):
    """Vectorised inverse: bytes uint8 [..., 12] -> codes uint8 [..., 32]."""
    c = np.empty(by.shape[:-1] + (32,), dtype=np.uint8)
    for b in range(4):
        spill = np.zeros(by.shape[:-1], dtype=np.uint8)
        for j in range(3):
            byte = by[..., 4 * j + b]
            c[..., 8 * j + b] = byte & 7
            c[..., 8 * j + 4 + b] = (byte >> 3) & 7
            spill |= ((byte >> 6) & 3) << (2 * j)
        c[..., 24 + b] = spill & 7
        c[..., 28 + b] = (spill >> 3) & 7
    return c


def _place(k: int, r, g):
    """Tile, row-in-tile, step, quad, group-in-quad and quads-in-step of (row r, group g)."""
    gp = layout(1, k)["padded_groups"]
    r = np.asarray(r, dtype=np.int64)
    g = np.asarray(g, dtype=np.int64)
    T, i = np.divmod(r, TILE_ROWS)
    s, u = np.divmod(g, STEP_GROUPS)
    kb, t = np.divmod(u, QUAD)
    q = np.minimum(STEP_GROUPS, gp - STEP_GROUPS * s) // QUAD
    return gp, T, i, s, kb, t, q


def word_offset(k: int, r, g, j):
    """Code-plane byte offset of word j (0..2) of group g of row r.

    Tile T = r // 16 starts at T * 192 * Gp.  Step s = g // 16 of a tile starts
    3072 * s bytes into it (all steps but the last hold 16 groups) and holds
    3 * 4q pieces of 16 bytes, q = p/4 quads of groups.  Piece 16*(q*j + kb) + i
    is word j of the quad kb (groups 16s+4kb .. 16s+4kb+3) of the tile's row
    i = r % 16; inside the piece, 4-byte word t belongs to group 16s+4kb+t.
    So word j of a step is one run of 64q bytes per quad index, rows innermost.
    """
    gp, T, i, s, kb, t, q = _place(k, r, g)
    return (T * TILE_ROWS * CODE_BYTES_PER_GROUP * gp + 3072 * s
            + 16 * (16 * (q * np.asarray(j) + kb) + i) + 4 * t)


def scale_offset(k: int, r, g):
    """Scale-plane byte offset of the scale of group g of row r.

    Tile T starts at T * 16 * Gp, step s at 256 * s inside it; within the step,
    byte 4*(16*kb + i) + t is the scale of group 16s+4kb+t of row i = r % 16.
    """
    gp, T, i, s, kb, t, q = _place(k, r, g)
    return T * TILE_ROWS * gp + 256 * s + 4 * (16 * kb + i) + t


def _code_index(k: int, rows) -> np.ndarray:
    """Plane byte of byte 4j+b of each real group's 12 packed bytes, [len(rows)][G][12]."""
    G = k // GROUP
    r = np.asarray(rows, dtype=np.int64)[:, None, None, None]
    g = np.arange(G)[None, :, None, None]
    j = np.arange(3)[None, None, :, None]
    b = np.arange(4)[None, None, None, :]
    return (word_offset(k, r, g, j) + b).reshape(len(rows), G, 12)


def _scale_index(k: int, rows) -> np.ndarray:
    G = k // GROUP
    return scale_offset(k, np.asarray(rows, dtype=np.int64)[:, None], np.arange(G)[None, :])


def pack(codes: np.ndarray, scales: np.ndarray, block: int = 1024):
    """codes uint8 [n][k] (only bits 0..2 used), scales uint8 [n][k/32] ->
    (code_plane uint8 [code_plane_bytes], scale_plane uint8 [scale_plane_bytes]),
    padding bytes zero.  Rows are placed `block` at a time to bound memory."""
    n, k = codes.shape
    L = layout(n, k)
    G = L["groups"]
    cp = np.zeros(L["code_plane_bytes"], dtype=np.uint8)
    sp = np.zeros(L["scale_plane_bytes"], dtype=np.uint8)
    for r0 in range(0, n, block):
        rows = np.arange(r0, min(n, r0 + block))
        cp[_code_index(k, rows).reshape(-1)] = _pack_bytes(codes[rows].reshape(len(rows), G, 32)).reshape(-1)
        sp[_scale_index(k, rows).reshape(-1)] = scales[rows].reshape(-1)
    return cp, sp


def unpack(code_plane: np.ndarray, scale_plane: np.ndarray, n: int, k: int, rows=None):
    """(code_plane, scale_plane) of an n x k matrix -> (codes uint8 [len(rows)][k],
    scales uint8 [len(rows)][k/32]) for `rows` (default: all n rows)."""
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    G = k // GROUP
    by = np.asarray(code_plane)[_code_index(k, rows)]
    return _unpack_bytes(by).reshape(len(rows), k), np.asarray(scale_plane)[_scale_index(k, rows)]


# ---------------------------------------------------------------- the layer

def dequantize(codes: np.ndarray, scales: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """w[n][k] = E4M3FN(codebook[n][codes[n][k] & 7]) * 2^(scales[n][k/32] - 127), float64."""
    n, k = codes.shape
    rows = np.arange(n)[:, None]
    cbv = E4M3FN_TABLE[codebook.astype(np.int64)]               # [n][8]
    w = cbv[rows, (codes & 7).astype(np.int64)]                  # [n][k]
    return w * np.repeat(e8m0_decode(scales), GROUP, axis=1)


def linear(code_plane, scale_plane, codebook, n, k, x_bits, rows=None, block=2048):
    """y[m][r] = sum_k x[m][k] w[r][k] and bound[m][r] = sum_k |x[m][k] w[r][k]|
    in float64, for r in `rows` (default: all n rows).  Weights are read back
    from the packed planes with this module's own unpacking, so a wrong
    packing shows up here.  Rows are processed in blocks of `block` to bound
    memory; the per-block products are plain fp64 matrix products."""
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    x = bf16_decode(x_bits)                                      # [m][k]
    xa = np.abs(x)
    y = np.empty((x.shape[0], rows.size), dtype=np.float64)
    bound = np.empty_like(y)
    for s in range(0, rows.size, block):
        r = rows[s:s + block]
        codes, scales = unpack(code_plane, scale_plane, n, k, rows=r)
        w = dequantize(codes, scales, codebook[r])
        y[:, s:s + r.size] = x @ w.T
        bound[:, s:s + r.size] = xa @ np.abs(w).T
    return y, bound


def within_tolerance(y_gpu, y_ref, bound, rel=1e-3):
    """Acceptance rule: |y - y_ref| <= rel * sum_k |x_k w_k|, and an exact 0
    where that sum is 0.  Returns (ok, worst err/bound ratio)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    zero = bound == 0
    ok = bool(np.all(err[~zero] <= rel * bound[~zero]) and np.all(y_gpu[zero] == 0))
    ratio = float(np.max(err[~zero] / bound[~zero])) if (~zero).any() else 0.0
    return ok, ratio


# --------------------------------------------------------------------- MoE

def topk_route(logits: np.ndarray, topk: int) -> np.ndarray:
    """Top-k expert ids per token by router logit, highest first; equal logits
    go to the lower expert index.  Softmax is monotone, so ranking the logits
    ranks the routing probabilities."""
    t, E = logits.shape
    ids = np.empty((t, topk), dtype=np.int32)
    for i in range(t):
        order = sorted(range(E), key=lambda e: (-float(logits[i, e]), e))
        ids[i] = order[:topk]
    return ids


def expert_union(ids: np.ndarray) -> np.ndarray:
    """Sorted distinct experts that at least one token picked."""
    return np.unique(ids.reshape(-1)).astype(np.int32)


def grouped_linear(planes, ids, x_bits, x_by_slot: bool, rows=None):
    """Expert-grouped products for one verify round.

    planes: list over experts of (code_plane, scale_plane, codebook, n, k).
    ids:    int [t][topk] routed experts.
    x_bits: bf16 [t][k] when x_by_slot is False (each token's activation goes to
            all of its experts), or bf16 [t][topk][k] when True (one activation
            per (token, slot), as for a down projection).
    Returns y[t][topk][n] and the matching bounds; each expert in the union is
    dequantised once and applied only to the (token, slot) pairs routed to it.
    """
    t, topk = ids.shape
    n = planes[0][3]
    nr = n if rows is None else len(rows)
    y = np.zeros((t, topk, nr))
    bound = np.zeros_like(y)
    for e in expert_union(ids):
        pairs = [(i, j) for i in range(t) for j in range(topk) if ids[i, j] == e]
        cp, sp, cb, ne, ke = planes[e]
        xs = np.stack([x_bits[i, j] if x_by_slot else x_bits[i] for i, j in pairs])
        ye, be = linear(cp, sp, cb, ne, ke, xs, rows=rows)
        for p, (i, j) in enumerate(pairs):
            y[i, j] = ye[p]
            bound[i, j] = be[p]
    return y, bound


def routing_mass(logits: np.ndarray) -> np.ndarray:
    """Total routing mass per expert: sum over tokens of softmax(logits[t])[e], fp64."""
    z = np.asarray(logits, dtype=np.float64)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    return p.sum(axis=0)


def budget_route(logits: np.ndarray, topk: int, budget: int):
    """Expert-budget routing of one verify round.

    Returns (experts, ids): the kept experts, ascending (int32 [budget]), and
    each token's top-k experts inside them, highest logit first (int32
    [t][topk]).  Requires topk <= budget <= number of experts."""
    t, E = logits.shape
    if not (1 <= topk <= budget <= E):
        raise ValueError("need 1 <= topk <= budget <= experts")
    mass = routing_mass(logits)
    order = sorted(range(E), key=lambda e: (-float(mass[e]), e))
    kept = sorted(order[:budget])
    ids = np.empty((t, topk), dtype=np.int32)
    for i in range(t):
        inside = sorted(kept, key=lambda e: (-float(logits[i, e]), e))
        ids[i] = inside[:topk]
    return np.array(kept, dtype=np.int32), ids


def silu(z):
    """z * sigmoid(z) = z / (1 + e^-z), fp64."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def combine_weights(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """p[t][s]: softmax over token t's routed logits logits[t][ids[t][s]], fp64."""
    sel = np.take_along_axis(np.asarray(logits, dtype=np.float64), np.asarray(ids, dtype=np.int64), axis=1)
    p = np.exp(sel - sel.max(axis=1, keepdims=True))
    return p / p.sum(axis=1, keepdims=True)


def moe_mlp(planes_gu, planes_dn, ids, logits, x_bits, rows=None):
    """Fused expert MLP of one verify round: out[t][r] = sum_s p[t][s] *
    sum_j w_dn[e][r][j] * silu(g[t][s][j]) * u[t][s][j], with g and u the gate
    and up halves of expert e = ids[t][s] applied to x[t].

    planes_gu / planes_dn: lists over experts of (code_plane, scale_plane,
    codebook, n, k); gate/up has n = 2I, down has k = I.  Returns out[t][nr]
    and the first-order bound of each output (module header), for the down
    rows `rows` (default: all)."""
    t, topk = ids.shape
    I = planes_gu[0][3] // 2
    n_dn = planes_dn[0][3]
    rows = np.arange(n_dn) if rows is None else np.asarray(rows, dtype=np.int64)
    gu, bgu = grouped_linear(planes_gu, ids, x_bits, False)          # [t][topk][2I]
    g, u = gu[..., :I], gu[..., I:]
    bg, bu = bgu[..., :I], bgu[..., I:]
    sg = 1.0 / (1.0 + np.exp(-g))
    h = g * sg * u
    dh_dg = sg * (1.0 + g * (1.0 - sg)) * u
    dh_du = g * sg
    slack = np.abs(h) + np.abs(dh_dg) * bg + np.abs(dh_du) * bu
    p = combine_weights(logits, ids)
    out = np.zeros((t, rows.size))
    bound = np.zeros_like(out)
    for e in expert_union(ids):
        cp, sp, cb, ne, ke = planes_dn[e]
        codes, scales = unpack(cp, sp, ne, ke, rows=rows)
        w = dequantize(codes, scales, cb[rows])                       # [nr][I]
        for i in range(t):
            for j in range(topk):
                if ids[i, j] == e:
                    out[i] += p[i, j] * (w @ h[i, j])
                    bound[i] += p[i, j] * (np.abs(w) @ slack[i, j])
    return out, bound
