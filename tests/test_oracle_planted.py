"""Planted mistakes in the draft-head, expert-budget, quantizer, codebook-fit
and fused-MLP oracles.  Each plant is one plausible slip -- a wrong tie rule, a
dropped or shifted scale, an off-by-one exponent, swapped halves, a missing
renormalisation, rounding half away from zero -- made on the CPU by replacing
one oracle function for the duration of the test, and each test checks that
an existing pin then fails.  A pin that kept passing with the mistake in place
would not have caught it.  (The 3.25-bit layer's own oracle has its planted
mistakes at the end of test_oracle.py.)"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import q2_head, q3_fit, q3_oracle, q3_quant

import test_oracle_budget as budget_pins
import test_oracle_fit as fit_pins
import test_oracle_head as head_pins
import test_oracle_moe_mlp as mlp_pins
import test_oracle_quant as quant_pins


def caught(pin, *args):
    """The pin fails (an assertion) with the planted mistake in place."""
    with pytest.raises(AssertionError):
        pin(*args)


def plant(monkeypatch, module, name, fn):
    """Replace module.name (and the package's re-export of it, if any)."""
    monkeypatch.setattr(module, name, fn)
    if getattr(oracle, name, None) is not None:
        monkeypatch.setattr(oracle, name, fn)


# ------------------------------------------------------------ two-bit draft head

def test_head_dropped_group_scale(monkeypatch):
    real = q2_head.dequantize2
    plant(monkeypatch, q2_head, "dequantize2", lambda codes, scales, cb4: real(codes, np.full_like(scales, 127), cb4))
    caught(head_pins.test_linear2_against_torch_decode)


def test_head_codebook_read_backwards(monkeypatch):
    real = q2_head.dequantize2
    plant(monkeypatch, q2_head, "dequantize2",
          lambda codes, scales, cb4: real(codes, scales, np.ascontiguousarray(np.asarray(cb4)[:, ::-1])))
    caught(head_pins.test_linear2_against_torch_decode)


def test_head_codes_in_the_wrong_bit_pairs(monkeypatch):
    # a packer that puts code 16j+4q+b into bits 2(3-q) instead of 2q of its byte
    real = q2_head.pack_group2

    def flipped(c):
        c = list(c)
        return real([c[16 * j + 4 * (3 - q) + b] for j in range(2) for q in range(4) for b in range(4)])
    plant(monkeypatch, q2_head, "pack_group2", flipped)
    caught(head_pins.test_group_words_hand_derived)


def test_head_shortlist_ties_to_the_higher_row(monkeypatch):
    def higher(scores, size=q2_head.SHORTLIST):
        scores = np.asarray(scores)
        idx = np.arange(scores.shape[1])
        return np.stack([np.lexsort((-idx, -s.astype(np.float64)))[:size] for s in scores]).astype(np.int32)
    plant(monkeypatch, q2_head, "shortlist", higher)
    caught(head_pins.test_shortlist_ties_and_brute_force)


def test_head_fp8_scale_off_by_one(monkeypatch):
    real = q2_head.mxfp8_dequantize
    plant(monkeypatch, q2_head, "mxfp8_dequantize", lambda e8, s8: real(e8, np.asarray(s8) + 1))
    caught(head_pins.test_mxfp8_and_rescore_against_torch)


def test_head_decision_ties_to_the_higher_row(monkeypatch):
    def higher(ids, scores8):
        ids = np.asarray(ids)
        return np.array([ids[i][max(range(ids.shape[1]), key=lambda j: (float(scores8[i][j]), int(ids[i][j])))]
                         for i in range(ids.shape[0])], dtype=np.int32)
    plant(monkeypatch, q2_head, "decide", higher)
    caught(head_pins.test_decide_brute_force)


# ------------------------------------------------------------ expert budget

def test_budget_mass_without_normalisation(monkeypatch):
    def unnormalised(logits):
        z = np.asarray(logits, dtype=np.float64)
        return np.exp(z - z.max(axis=1, keepdims=True)).sum(axis=0)
    plant(monkeypatch, q3_oracle, "routing_mass", unnormalised)
    caught(budget_pins.test_routing_mass_against_torch_softmax)
    caught(budget_pins.test_kept_set_brute_force)


def test_budget_kept_by_the_largest_share_instead_of_the_total(monkeypatch):
    def largest_share(logits):
        z = np.asarray(logits, dtype=np.float64)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        return (p / p.sum(axis=1, keepdims=True)).max(axis=0)
    plant(monkeypatch, q3_oracle, "routing_mass", largest_share)
    caught(budget_pins.test_kept_set_brute_force)


def test_budget_ties_to_the_higher_expert(monkeypatch):
    def higher(logits, topk, budget):
        t, E = logits.shape
        mass = q3_oracle.routing_mass(logits)
        kept = sorted(sorted(range(E), key=lambda e: (-float(mass[e]), -e))[:budget])
        ids = np.array([sorted(kept, key=lambda e: (-float(logits[i, e]), -e))[:topk] for i in range(t)],
                       dtype=np.int32)
        return np.array(kept, dtype=np.int32), ids
    plant(monkeypatch, q3_oracle, "budget_route", higher)
    caught(budget_pins.test_equal_logits_go_to_the_lower_expert)


# ------------------------------------------------------------ quantizer

def test_quant_code_ties_to_the_higher_index(monkeypatch):
    def higher(w, codebook, scales):
        w = np.asarray(w, dtype=np.float32).astype(np.float64)
        n, k = w.shape
        e = np.repeat(np.asarray(scales, dtype=np.int64) - 127, 32, axis=1)
        v = q3_quant.codebook_values(codebook)
        out = np.empty((n, k), dtype=np.uint8)
        for r in range(n):
            for c in range(k):
                d = [abs(w[r, c] - np.ldexp(v[r, j], int(e[r, c]))) for j in range(8)]
                out[r, c] = max(range(8), key=lambda j: (-d[j], j))     # equal distance: the higher index
        return out
    plant(monkeypatch, q3_quant, "snap", higher)
    caught(quant_pins.test_ties_go_to_the_lower_index)


def test_quant_scale_one_too_large(monkeypatch):
    real = q3_quant.choose_scales
    plant(monkeypatch, q3_quant, "choose_scales",
          lambda w, codebook: np.minimum(real(w, codebook).astype(np.int64) + 1, 254).astype(np.uint8))
    caught(quant_pins.test_scale_rule_edges)
    caught(quant_pins.test_random_matches_rational_brute_force, 0)


def test_quant_scale_needs_strict_room(monkeypatch):
    # "max |w| < cbmax * 2^(s-127)" instead of "<=": a group that fits exactly gets one scale too many
    def strict(w, codebook):
        w = np.asarray(w, dtype=np.float32)
        n, k = w.shape
        amax = np.abs(w.astype(np.float64)).reshape(n, k // 32, 32).max(axis=2)
        cbmax = np.abs(q3_quant.codebook_values(codebook)).max(axis=1)[:, None]
        s = np.full(amax.shape, 254, dtype=np.int64)
        for cand in range(254, -1, -1):
            s = np.where(amax < np.ldexp(cbmax, cand - 127), cand, s)
        return s.astype(np.uint8)
    plant(monkeypatch, q3_quant, "choose_scales", strict)
    caught(quant_pins.test_scale_rule_edges)


# ------------------------------------------------------------ codebook fit

def test_fit_exponent_of_exact_powers_of_two(monkeypatch):
    def frexp_only(w):
        w = np.asarray(w, dtype=np.float32).astype(np.float64)
        n, k = w.shape
        amax = np.abs(w).reshape(n, k // 32, 32).max(axis=2)
        _, x = np.frexp(amax)                       # forgets that f == 0.5 needs one less
        return np.where(amax == 0, 0, x).astype(np.int64)
    plant(monkeypatch, q3_fit, "group_exponents", frexp_only)
    caught(fit_pins.test_group_exponents_match_frexp)


def test_fit_grid_rounds_half_away_from_zero(monkeypatch):
    def away(w):
        w = np.asarray(w, dtype=np.float32).astype(np.float64)
        e = np.repeat(q3_fit.group_exponents(w), 32, axis=1)
        v = np.ldexp(w, q3_fit.GRID_BITS - e)
        return (np.sign(v) * np.floor(np.abs(v) + 0.5)).astype(np.int64)
    plant(monkeypatch, q3_fit, "grid_values", away)
    caught(fit_pins.test_grid_values_are_exact_rounding_half_even)


def test_fit_e4m3_ties_away_from_zero(monkeypatch):
    def away(value):
        mag = abs(value)
        best = None
        for b, v in q3_fit.E4M3FN_POSITIVE:
            d = abs(mag - v)
            if best is None or d <= best[0]:        # equal distances: the larger value
                best = (d, b)
        return best[1] | (0x80 if value < 0 else 0)
    plant(monkeypatch, q3_fit, "round_e4m3fn", away)
    caught(fit_pins.test_e4m3_rounding_matches_torch_on_dyadic_values)


def test_fit_nearest_ties_to_the_higher_centroid(monkeypatch):
    def higher(q, cents):
        best = np.zeros(q.shape, dtype=np.int64)
        bs = np.full(q.shape, cents[0][0], dtype=np.int64)
        bc = np.full(q.shape, cents[0][1], dtype=np.int64)
        for j in range(1, len(cents)):
            s, c = cents[j]
            closer = np.abs(q * c - s) * bc <= np.abs(q * bc - bs) * c
            best = np.where(closer, j, best)
            bs = np.where(closer, s, bs)
            bc = np.where(closer, c, bc)
        return best
    plant(monkeypatch, q3_fit, "nearest", higher)
    caught(fit_pins.test_nearest_equal_distances_go_to_the_lower_centroid)
    caught(fit_pins.test_lloyd_updates_match_brute_force, 7, 256)


def test_fit_cluster_means_rounded_to_integers(monkeypatch):
    # a Lloyd step that stores each centroid as its integer-rounded mean instead of the exact rational
    real = q3_fit.nearest

    def lloyd(q, trace=None):
        q = np.asarray(q, dtype=np.int64)
        cents = q3_fit.initial_centroids(q)
        for _ in range(q3_fit.MAX_UPDATES):
            idx = real(q, cents)
            new = [(int(round(Fraction(int(q[idx == j].sum()), int((idx == j).sum())))), 1) if (idx == j).any()
                   else cents[j] for j in range(8)]
            new = [new[j] for j in sorted(range(8), key=lambda j: (Fraction(*new[j]), j))]
            if trace is not None:
                trace.append(list(new))
            same = new == cents
            cents = new
            if same:
                break
        return cents
    plant(monkeypatch, q3_fit, "lloyd", lloyd)
    caught(fit_pins.test_lloyd_updates_match_brute_force, 6, 96)


# ------------------------------------------------------------ fused expert MLP

def test_mlp_combine_without_renormalisation(monkeypatch):
    def raw(logits, ids):
        z = np.asarray(logits, dtype=np.float64)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        return np.take_along_axis(p, np.asarray(ids, dtype=np.int64), axis=1)   # full-softmax shares as they are
    plant(monkeypatch, q3_oracle, "combine_weights", raw)
    caught(mlp_pins.test_combine_weights_renormalise_the_full_softmax)
    caught(mlp_pins.test_matches_torch_composition)


def test_mlp_gate_and_up_halves_swapped(monkeypatch):
    real = q3_oracle.grouped_linear

    def swapped(planes, ids, x_bits, x_by_slot, rows=None):
        y, b = real(planes, ids, x_bits, x_by_slot, rows)
        half = y.shape[-1] // 2
        return np.concatenate([y[..., half:], y[..., :half]], -1), np.concatenate([b[..., half:], b[..., :half]], -1)
    plant(monkeypatch, q3_oracle, "grouped_linear", swapped)
    caught(mlp_pins.test_matches_torch_composition)


def test_mlp_silu_with_the_wrong_sign(monkeypatch):
    plant(monkeypatch, q3_oracle, "silu", lambda z: np.asarray(z, np.float64) / (1.0 + np.exp(np.asarray(z, np.float64))))
    caught(mlp_pins.test_silu_and_bound_derivatives_against_autograd)
