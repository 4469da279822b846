"""Pins of the expert-budget routing oracle (Hibana page, "Adaptive speculation"
/ "Expert sharing"): the page's toy figure reproduced by a hand-built round,
brute force over expert subsets and per-token ranking, the reduction to plain
top-k when the budget covers every expert, and torch's softmax for the mass."""
import itertools

import numpy as np
import torch

import oracle
from conftest import read_golden

GOLD = read_golden("expert_budget_toy.txt")


def _rows(tag):
    return [[int(v) for v in r.split()[1:]] for r in GOLD if r.split()[0] == tag]


def _toy():
    logits = np.zeros((6, 12), dtype=np.float32)
    for t, first, second in _rows("token"):
        logits[t, first] = 4.0
        logits[t, second] = 2.0
    return logits


def test_toy_figure_numbers():
    logits = _toy()
    kept, ids = oracle.budget_route(logits, 2, 4)
    assert kept.tolist() == _rows("kept")[0]
    for t, a, b in _rows("route"):
        assert ids[t].tolist() == [a, b]
    plain = oracle.topk_route(logits, 2)
    assert len(oracle.expert_union(plain)) == _rows("plain_union")[0][0]          # 8 experts without a budget
    assert len(oracle.expert_union(ids)) == _rows("loaded")[0][0] == 4             # 4 of 12 read
    assert len(oracle.expert_union(ids)) / len(oracle.expert_union(plain)) == 0.5  # 50% of the bytes
    keep = sum(set(ids[t]) == set(plain[t]) for t in range(6))
    assert keep == _rows("keep_own")[0][0]                                          # 2 of 6 keep their top-2
    assert all(ids[t, 0] == plain[t, 0] for t in range(6))                          # only second choices replaced


def test_budget_covering_every_expert_is_plain_topk():
    rng = np.random.default_rng(0)
    logits = rng.standard_normal((8, 64)).astype(np.float32)
    kept, ids = oracle.budget_route(logits, 8, 64)
    assert kept.tolist() == list(range(64))
    assert np.array_equal(ids, oracle.topk_route(logits, 8))


def test_kept_set_brute_force():
    rng = np.random.default_rng(1)
    for E, B, k, t in [(6, 3, 2, 4), (8, 4, 2, 5), (7, 5, 3, 3), (8, 2, 1, 6)]:
        logits = rng.standard_normal((t, E)).astype(np.float32)
        kept, ids = oracle.budget_route(logits, k, B)
        z = np.exp(logits.astype(np.float64) - logits.max(axis=1, keepdims=True))
        mass = (z / z.sum(axis=1, keepdims=True)).sum(axis=0)
        best = max(itertools.combinations(range(E), B), key=lambda S: sum(mass[e] for e in S))
        assert kept.tolist() == list(best)
        for i in range(t):
            want = sorted(best, key=lambda e: -logits[i, e])[:k]
            assert ids[i].tolist() == want


def test_routing_mass_against_torch_softmax():
    rng = np.random.default_rng(2)
    logits = (3 * rng.standard_normal((8, 64))).astype(np.float32)
    m = oracle.routing_mass(logits)
    ref = torch.softmax(torch.from_numpy(logits).double(), dim=1).sum(0).numpy()
    assert np.allclose(m, ref, rtol=0, atol=1e-14)
    assert abs(m.sum() - 8.0) < 1e-12      # every token's mass sums to one


def test_equal_logits_go_to_the_lower_expert():
    logits = np.zeros((2, 6), dtype=np.float32)      # every expert ties
    kept, ids = oracle.budget_route(logits, 2, 3)
    assert kept.tolist() == [0, 1, 2]
    assert ids.tolist() == [[0, 1], [0, 1]]
