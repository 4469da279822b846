"""Seeded synthetic inputs for the 3-bit FP8-codebook linear layer.

This module only draws random numbers and rounds them to the storage types
(E4M3FN bytes, bf16 bits) with torch's CPU casts; it holds none of the
layer's arithmetic (no packing, no decoding, no products).  Both the CPU
oracle's tests and the GPU path are fed from here, so the two sides see the
same inputs without sharing any code.

Distributions (one per tensor, all seeded):
  * codes:      uint8 [n][k], i.i.d. uniform over 0..7
  * codebook:   uint8 [n][8], per output row 8 draws of N(0,1) rounded
                (round-to-nearest-even) to OCP E4M3FN
  * scales:     uint8 [n][k/32], biased exponent 127+e with e uniform over the
                integers -10..-4 (a power-of-two scale per 32-weight group)
  * x:          uint16 [m][k], bf16 bit patterns of N(0,1) draws (RNE)
  * logits:     float32 [t][E], N(0,1) (MoE router scores)
  Two-bit draft head (make_head): codes uniform over 0..3, a 4-entry E4M3FN
  codebook per row from N(0,1), scales as above; the FP8 head's elements are
  N(0,1) draws rounded to E4M3FN with one scale byte per 32 drawn like the
  group scales; the two heads are drawn independently.

Each tensor gets its own child stream of numpy's PCG64, spawned from
SeedSequence(seed) in a fixed order, so a tensor never depends on the shape
of another.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np
import torch

SCALE_EXP_LO = -10
SCALE_EXP_HI = -4
SCALE_BIAS = 127


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def round_to_e4m3fn_bytes(values: np.ndarray) -> np.ndarray:
    """float values -> OCP E4M3FN bytes, round-to-nearest-even (torch CPU cast)."""
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32))
    b = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    if ((b & 0x7F) == 0x7F).any():
        raise ValueError("codebook draw outside the finite E4M3FN range")
    return b


def round_to_bf16_bits(values: np.ndarray) -> np.ndarray:
    """float values -> bf16 bit patterns (uint16), round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def draw_codes(rng, n, k):
    return rng.integers(0, 8, size=(n, k), dtype=np.uint8)


def draw_codebook(rng, n):
    return round_to_e4m3fn_bytes(rng.standard_normal((n, 8)))


def draw_scales(rng, n, k):
    e = rng.integers(SCALE_EXP_LO, SCALE_EXP_HI + 1, size=(n, k // 32))
    return (SCALE_BIAS + e).astype(np.uint8)


def draw_x(rng, m, k):
    return round_to_bf16_bits(rng.standard_normal((m, k)))


@dataclass
class Layer:
    """One unpacked linear layer: w[n][k] = E4M3(codebook[n][codes[n][k]]) * 2^(scales[n][k/32]-127)."""
    n: int
    k: int
    codes: np.ndarray      # uint8 [n][k]
    codebook: np.ndarray   # uint8 [n][8]
    scales: np.ndarray     # uint8 [n][k/32]


def make_layer(n: int, k: int, seed: int = 0, stream_offset: int = 0) -> Layer:
    rs = _streams(seed, stream_offset + 3)[stream_offset:]
    return Layer(n, k, draw_codes(rs[0], n, k), draw_codebook(rs[1], n), draw_scales(rs[2], n, k))


def make_linear(n: int, k: int, m: int, seed: int = 0):
    """A layer and bf16 activations x[m][k]; streams in the order codes, codebook, scales, x."""
    rs = _streams(seed, 4)
    layer = Layer(n, k, draw_codes(rs[0], n, k), draw_codebook(rs[1], n), draw_scales(rs[2], n, k))
    return layer, draw_x(rs[3], m, k)


def make_layer_on_device(n: int, k: int, m: int, seed: int = 0, device: str = "cuda"):
    """A layer too large to draw on the host: codes uint8 [n][k] drawn on the
    device (torch's generator there, seeded, uniform over 0..7, a torch tensor),
    the codebook, scales and bf16 activations x[m][k] drawn as in make_linear
    (numpy arrays).  Returns (codes, codebook, scales, x)."""
    rs = _streams(seed, 4)
    g = torch.Generator(device=device)
    g.manual_seed(int(rs[0].integers(0, 2 ** 63 - 1)))
    codes = torch.randint(0, 8, (n, k), dtype=torch.uint8, device=device, generator=g)
    return codes, draw_codebook(rs[1], n), draw_scales(rs[2], n, k), draw_x(rs[3], m, k)


@dataclass
class MoEInputs:
    experts_gu: list = field(default_factory=list)   # Layer per expert (gate/up)
    experts_dn: list = field(default_factory=list)   # Layer per expert (down)
    logits: np.ndarray = None                        # float32 [t][E]
    x: np.ndarray = None                             # bf16 bits [t][k_gu]
    x_dn: np.ndarray = None                          # bf16 bits [t][topk][k_dn]


def make_moe(num_experts=64, k_gu=2048, n_gu=1536, k_dn=768, n_dn=2048, tokens=8, topk=8,
             seed: int = 0) -> MoEInputs:
    """Expert-grouped verify round: per expert a gate/up and a down matrix,
    router logits, the tokens' activations and an independent activation per
    (token, slot) for the down projection."""
    rs = _streams(seed, 6 * num_experts + 3)
    out = MoEInputs()
    for e in range(num_experts):
        a = rs[6 * e: 6 * e + 6]
        out.experts_gu.append(Layer(n_gu, k_gu, draw_codes(a[0], n_gu, k_gu), draw_codebook(a[1], n_gu),
                                    draw_scales(a[2], n_gu, k_gu)))
        out.experts_dn.append(Layer(n_dn, k_dn, draw_codes(a[3], n_dn, k_dn), draw_codebook(a[4], n_dn),
                                    draw_scales(a[5], n_dn, k_dn)))
    t = rs[6 * num_experts:]
    out.logits = t[0].standard_normal((tokens, num_experts)).astype(np.float32)
    out.x = draw_x(t[1], tokens, k_gu)
    out.x_dn = draw_x(t[2], tokens * topk, k_dn).reshape(tokens, topk, k_dn)
    return out


def digest(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        a = np.ascontiguousarray(a)
        h.update(str(a.dtype).encode())
        h.update(str(a.shape).encode())
        h.update(a.tobytes())
    return h.hexdigest()[:16]


@dataclass
class Head:
    """A two-bit draft head and its FP8 (MXFP8) counterpart, unpacked.
    w2[n][k] = E4M3(cb4[n][codes[n][k]]) * 2^(scales[n][k/32]-127);
    w8[n][k] = E4M3(e8[n][k]) * 2^(s8[n][k/32]-127)."""
    n: int
    k: int
    codes: np.ndarray      # uint8 [n][k], 0..3
    codebook: np.ndarray   # uint8 [n][4]
    scales: np.ndarray     # uint8 [n][k/32]
    e8: np.ndarray         # uint8 [n][k]
    s8: np.ndarray         # uint8 [n][k/32]


def make_head(n: int, k: int, m: int, seed: int = 0):
    """A draft head and bf16 activations x[m][k]; streams in the order codes,
    codebook, scales, FP8 elements, FP8 scales, x.  The FP8 elements are drawn
    in row blocks (the same numbers as one draw, less memory)."""
    rs = _streams(seed, 6)
    e8 = np.empty((n, k), dtype=np.uint8)
    block = max(1, (1 << 25) // k)
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        e8[r0:r1] = round_to_e4m3fn_bytes(rs[3].standard_normal((r1 - r0, k)))
    head = Head(n, k, rs[0].integers(0, 4, size=(n, k), dtype=np.uint8),
                round_to_e4m3fn_bytes(rs[1].standard_normal((n, 4))), draw_scales(rs[2], n, k),
                e8, draw_scales(rs[4], n, k))
    return head, draw_x(rs[5], m, k)


def make_quant(n: int, k: int, seed: int = 0):
    """Weights to quantize and their per-row codebooks: w float32 [n][k] drawn
    N(0,1) * 2^u with u an integer per group of 32, uniform in [-12, 3] (so
    the groups' scales spread), and E4M3FN codebooks [n][8] drawn as for a
    layer.  Streams in the order codebook, group exponents, weights."""
    rs = _streams(seed, 3)
    codebook = draw_codebook(rs[0], n)
    u = rs[1].integers(-12, 4, size=(n, k // 32))
    w = rs[2].standard_normal((n, k)) * np.repeat(np.ldexp(1.0, u), 32, axis=1)
    return w.astype(np.float32), codebook
