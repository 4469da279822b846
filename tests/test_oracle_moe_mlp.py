"""Pins of the fused expert-MLP oracle (Hibana page, "Adaptive speculation" /
"Expert sharing": the experts a verify round reads, run as SwiGLU MLPs and
combined by routing weight).  Pinned to a closed form on constant weights, to
an independent torch float64 composition (torch's E4M3FN decoding and ldexp,
F.silu, a full softmax renormalised over the routed experts), and the bound's
derivatives to torch autograd."""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle
import synth


def _planes(layers):
    return [(*oracle.pack(L.codes, L.scales), L.codebook, L.n, L.k) for L in layers]


def _const_layer(n, k, scale_byte):
    """Every weight = 2^(scale_byte - 127): codebook all 1.0 (0x38), codes 0..7 cycling."""
    codes = (np.arange(n * k) % 8).astype(np.uint8).reshape(n, k)
    return synth.Layer(n, k, codes, np.full((n, 8), 0x38, np.uint8), np.full((n, k // 32), scale_byte, np.uint8))


def test_closed_form_constant_weights():
    # Two experts, I = 32, K = 64, down to 24 rows; x = 1 everywhere.  Expert 0
    # has every weight 1, expert 1 every weight 2 (gate/up) and 1/2 (down).
    I, K, H = 32, 64, 24
    gu = [_const_layer(2 * I, K, 127), _const_layer(2 * I, K, 128)]
    dn = [_const_layer(H, I, 127), _const_layer(H, I, 126)]
    x = np.full((1, K), 0x3F80, np.uint16)                       # bf16 1.0
    ids = np.array([[1, 0]], dtype=np.int32)
    logits = np.array([[0.25, 1.5]], dtype=np.float32)           # expert 0: 0.25, expert 1: 1.5
    out, bound = oracle.moe_mlp(_planes(gu), _planes(dn), ids, logits, x)
    silu = lambda z: z / (1 + math.exp(-z))
    y0 = I * 1.0 * silu(64.0) * 64.0                              # g = u = 64
    y1 = I * 0.5 * silu(128.0) * 128.0                            # g = u = 128
    p1 = math.exp(1.5) / (math.exp(1.5) + math.exp(0.25))
    want = p1 * y1 + (1 - p1) * y0
    assert np.allclose(out, want, rtol=1e-14, atol=0)
    assert np.all(bound >= np.abs(out))


def _torch_reference(moe, ids, logits):
    """Independent composition: torch-decoded weights, F.silu, full softmax renormalised."""
    def deq(L):
        cb = torch.from_numpy(L.codebook).view(torch.float8_e4m3fn).to(torch.float64)
        w = torch.gather(cb, 1, torch.from_numpy(L.codes.astype(np.int64) & 7))
        e = torch.from_numpy(L.scales.astype(np.int64) - 127).repeat_interleave(32, dim=1)
        return torch.ldexp(w, e.to(torch.float64))
    x = torch.from_numpy(moe.x.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    full = torch.softmax(torch.from_numpy(logits).to(torch.float64), dim=1)
    t, topk = ids.shape
    out = torch.zeros(t, moe.experts_dn[0].n, dtype=torch.float64)
    for i in range(t):
        sel = full[i, torch.from_numpy(ids[i].astype(np.int64))]
        p = sel / sel.sum()
        for j in range(topk):
            e = int(ids[i, j])
            wgu = deq(moe.experts_gu[e])
            I = wgu.shape[0] // 2
            hid = F.silu(wgu[:I] @ x[i]) * (wgu[I:] @ x[i])
            out[i] += p[j] * (deq(moe.experts_dn[e]) @ hid)
    return out.numpy()


def test_matches_torch_composition():
    moe = synth.make_moe(num_experts=6, k_gu=64, n_gu=64, k_dn=32, n_dn=40, tokens=3, topk=2, seed=11)
    ids = oracle.topk_route(moe.logits, 2)
    out, bound = oracle.moe_mlp(_planes(moe.experts_gu), _planes(moe.experts_dn), ids, moe.logits, moe.x)
    ref = _torch_reference(moe, ids, moe.logits)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # row subset gives the same rows
    rows = np.array([0, 7, 39])
    sub, _ = oracle.moe_mlp(_planes(moe.experts_gu), _planes(moe.experts_dn), ids, moe.logits, moe.x, rows=rows)
    assert np.allclose(sub, out[:, rows], rtol=1e-14, atol=0)


def test_gate_and_up_halves_are_not_interchangeable():
    # silu(g)*u != silu(u)*g: swapping the halves of the gate/up rows must change the result
    moe = synth.make_moe(num_experts=2, k_gu=32, n_gu=64, k_dn=32, n_dn=8, tokens=2, topk=1, seed=5)
    ids = np.array([[0], [1]], dtype=np.int32)
    out, _ = oracle.moe_mlp(_planes(moe.experts_gu), _planes(moe.experts_dn), ids, moe.logits, moe.x)
    swapped = []
    for L in moe.experts_gu:
        perm = np.r_[32:64, 0:32]
        swapped.append(synth.Layer(L.n, L.k, L.codes[perm], L.codebook[perm], L.scales[perm]))
    out_s, _ = oracle.moe_mlp(_planes(swapped), _planes(moe.experts_dn), ids, moe.logits, moe.x)
    assert not np.allclose(out, out_s)
    assert np.allclose(out, _torch_reference(moe, ids, moe.logits), rtol=1e-12)


def test_combine_weights_renormalise_the_full_softmax():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((5, 16)).astype(np.float32)
    ids = oracle.topk_route(logits, 4)
    p = oracle.combine_weights(logits, ids)
    full = torch.softmax(torch.from_numpy(logits).double(), 1).numpy()
    sel = np.take_along_axis(full, ids.astype(np.int64), 1)
    assert np.allclose(p, sel / sel.sum(1, keepdims=True), rtol=1e-14)
    assert np.allclose(p.sum(1), 1.0)


def test_silu_and_bound_derivatives_against_autograd():
    z = np.linspace(-30, 30, 121)
    assert np.allclose(oracle.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-300)
    assert oracle.silu(0.0) == 0.0
    # The bound's sensitivities are |dh/dg| and |dh/du| of h = silu(g) * u: check them
    # through the bound of a single-expert round with all |w_dn| = 1 and one token.
    moe = synth.make_moe(num_experts=1, k_gu=32, n_gu=64, k_dn=32, n_dn=1, tokens=1, topk=1, seed=2)
    ones = synth.Layer(1, 32, np.zeros((1, 32), np.uint8), np.full((1, 8), 0x38, np.uint8),
                       np.full((1, 1), 127, np.uint8))
    ids = np.zeros((1, 1), np.int32)
    _, bound = oracle.moe_mlp(_planes(moe.experts_gu), _planes([ones]), ids, moe.logits, moe.x)
    gu, bgu = oracle.grouped_linear(_planes(moe.experts_gu), ids, moe.x, False)
    g = torch.tensor(gu[0, 0, :32], requires_grad=True)
    u = torch.tensor(gu[0, 0, 32:], requires_grad=True)
    h = F.silu(g) * u
    dg, du = torch.autograd.grad(h.sum(), (g, u))
    want = np.sum(np.abs(h.detach().numpy()) + np.abs(dg.numpy()) * bgu[0, 0, :32] + np.abs(du.numpy()) * bgu[0, 0, 32:])
    assert np.isclose(bound[0, 0], want, rtol=1e-12)
