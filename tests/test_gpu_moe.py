"""GPU parity of the MoE verify round: top-k routing (exact ids) and the
expert-grouped products against the oracle's routing and per-pair products."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q3():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_fp8_codebook_amd as q3
    q3.lib()
    return q3


@pytest.mark.parametrize("t,E,topk", [(8, 64, 8), (1, 10, 3), (5, 1024, 16), (3, 100, 100), (64, 128, 1)])
def test_topk_matches_oracle(q3, t, E, topk):
    logits = np.random.default_rng(E + t).standard_normal((t, E)).astype(np.float32)
    logits[0, :5] = 0.5          # ties go to the lower index
    ids = q3.q3_moe_topk(dev(logits), topk).cpu().numpy()
    assert np.array_equal(ids, oracle.topk_route(logits, topk))


def stack_experts(q3, layers):
    L = layers[0]
    st = q3.empty_stack(len(layers), L.n, L.k, "cuda")
    for e, layer in enumerate(layers):
        q3.q3_pack(dev(layer.codes), dev(layer.scales), dev(layer.codebook), out=st.expert(e))
    return st


def planes(layers):
    return [(*oracle.pack(L.codes, L.scales), L.codebook, L.n, L.k) for L in layers]


def run_round(q3, moe, topk, rows_gu=None, rows_dn=None):
    t = moe.logits.shape[0]
    ids_d = q3.q3_moe_topk(dev(moe.logits), topk)
    ids = ids_d.cpu().numpy()
    ref_ids = oracle.topk_route(moe.logits, topk)
    assert np.array_equal(ids, ref_ids)
    st_gu = stack_experts(q3, moe.experts_gu)
    st_dn = stack_experts(q3, moe.experts_dn)
    y_gu = q3.q3_grouped_expert_gemv(st_gu, dev(moe.x), ids_d, False).cpu().numpy()
    x_dn = np.ascontiguousarray(moe.x_dn[:, :topk]).reshape(t * topk, -1)
    y_dn = q3.q3_grouped_expert_gemv(st_dn, dev(x_dn), ids_d, True).cpu().numpy()
    ref_gu, b_gu = oracle.grouped_linear(planes(moe.experts_gu), ref_ids, moe.x, False, rows=rows_gu)
    ref_dn, b_dn = oracle.grouped_linear(planes(moe.experts_dn), ref_ids, moe.x_dn[:, :topk], True, rows=rows_dn)
    y_gu = y_gu.reshape(t, topk, -1)
    y_dn = y_dn.reshape(t, topk, -1)
    if rows_gu is not None:
        y_gu = y_gu[:, :, rows_gu]
        y_dn = y_dn[:, :, rows_dn]
    assert_close(y_gu.reshape(t * topk, -1), ref_gu.reshape(t * topk, -1), b_gu.reshape(t * topk, -1), "gate/up")
    assert_close(y_dn.reshape(t * topk, -1), ref_dn.reshape(t * topk, -1), b_dn.reshape(t * topk, -1), "down")
    return oracle.expert_union(ref_ids)


def test_grouped_small(q3):
    moe = synth.make_moe(num_experts=16, k_gu=256, n_gu=96, k_dn=96, n_dn=130, tokens=8, topk=4, seed=3)
    run_round(q3, moe, 4)


def test_grouped_one_token_many_experts(q3):
    moe = synth.make_moe(num_experts=12, k_gu=512, n_gu=64, k_dn=64, n_dn=48, tokens=1, topk=12, seed=4)
    run_round(q3, moe, 12)


def test_grouped_config2_full_size(q3):
    """64 experts, gate/up 2048->1536, down 768->2048, 8 drafted tokens x top-8."""
    moe = synth.make_moe(seed=0)
    rng = np.random.default_rng(2)
    rows_gu = np.sort(rng.choice(1536, 48, replace=False))
    rows_dn = np.sort(rng.choice(2048, 48, replace=False))
    u = run_round(q3, moe, 8, rows_gu, rows_dn)
    assert 20 <= u.size <= 64


# Expert-budget routing (Hibana page, "Adaptive speculation" / "Expert
# sharing").  The kept set is decided on fp32 routing masses on the GPU and on
# fp64 masses in the oracle: where the oracle's masses separate the budget-th
# and the next expert by more than the fp32 rounding allowance the two must
# agree exactly; otherwise the GPU's set must be valid against the fp64 masses
# within that allowance.  Inside the kept set the ranking compares the fp32
# logits themselves, so the routes are exact given the set.
def _budget_gpu(q3, logits, topk, budget):
    ids, kept = q3.q3_moe_budget_topk(dev(logits), topk, budget)
    return ids.cpu().numpy(), kept.cpu().numpy()


def _routes_inside(logits, kept, topk):
    """Plain numpy ranking of each token's logits over a given kept set (logit
    desc, expert asc)."""
    kept = np.asarray(kept)
    out = []
    for row in logits:
        order = np.lexsort((kept, -row[kept].astype(np.float64)))
        out.append(kept[order[:topk]])
    return np.array(out, dtype=np.int32)


def _check_budget(logits, topk, budget, ids, kept):
    t, E = logits.shape
    mass = oracle.routing_mass(logits)
    # fp32 mass on the GPU: each probability carries the error of its exp and of
    # the token's exp-sum (E/64 lane terms and a 6-level tree), and the mass sums
    # t of them in order: a generous 32 ulp per step of that chain.
    tol = 2e-6 * (t + E / 64 + 8) * mass.max()
    assert kept.shape == (budget,) and np.all(np.diff(kept) > 0) and kept.min() >= 0
    assert kept.max() < logits.shape[1]
    assert np.array_equal(ids, _routes_inside(logits, kept, topk))
    inside = np.zeros(mass.size, bool)
    inside[kept] = True
    if budget < mass.size:
        assert mass[inside].min() >= mass[~inside].max() - tol
        srt = np.sort(mass)[::-1]
        clear = srt[budget - 1] - srt[budget] > 2 * tol
    else:
        clear = True
    if clear:
        want_kept, want_ids = oracle.budget_route(logits, topk, budget)
        assert np.array_equal(kept, want_kept)
        assert np.array_equal(ids, want_ids)
    return clear


def test_budget_toy_figure(q3):
    from conftest import read_golden
    gold = read_golden("expert_budget_toy.txt")
    rows = lambda tag: [[int(v) for v in r.split()[1:]] for r in gold if r.split()[0] == tag]
    logits = np.zeros((6, 12), dtype=np.float32)
    for t, first, second in rows("token"):
        logits[t, first], logits[t, second] = 4.0, 2.0
    ids, kept = _budget_gpu(q3, logits, 2, 4)
    assert kept.tolist() == rows("kept")[0]
    for t, a, b in rows("route"):
        assert ids[t].tolist() == [a, b]
    assert np.unique(ids).size == rows("loaded")[0][0]


@pytest.mark.parametrize("t,E,topk,budget", [(8, 64, 8, 16), (8, 64, 8, 8), (8, 64, 8, 24), (8, 64, 2, 63),
                                             (1, 10, 3, 5), (64, 128, 1, 4), (5, 1024, 16, 100),
                                             (300, 256, 8, 32), (1024, 8, 2, 3), (2, 1000, 7, 999)])
def test_budget_matches_oracle(q3, t, E, topk, budget):
    clear = 0
    for seed in range(3):
        logits = np.random.default_rng(100 * seed + E + t).standard_normal((t, E)).astype(np.float32)
        ids, kept = _budget_gpu(q3, logits, topk, budget)
        clear += _check_budget(logits, topk, budget, ids, kept)
    assert clear >= 1                                # at least one round is decided exactly


def test_budget_config2_rounds(q3):
    """64 experts, 8 drafted tokens, top-8, budgets 8..64 on the MoE inputs' logits."""
    moe = synth.make_moe(seed=0)
    for budget in (8, 12, 16, 24, 32, 64):
        ids, kept = _budget_gpu(q3, moe.logits, 8, budget)
        _check_budget(moe.logits, 8, budget, ids, kept)
        assert np.unique(ids).size <= budget


def test_budget_equal_logits_go_to_lower_experts(q3):
    logits = np.full((4, 40), 0.25, dtype=np.float32)
    ids, kept = _budget_gpu(q3, logits, 3, 7)
    assert kept.tolist() == list(range(7))
    assert np.array_equal(ids, np.tile(np.arange(3, dtype=np.int32), (4, 1)))


def test_budget_covering_every_expert_is_plain_topk(q3):
    logits = np.random.default_rng(5).standard_normal((8, 64)).astype(np.float32)
    ids, kept = _budget_gpu(q3, logits, 8, 64)
    assert kept.tolist() == list(range(64))
    assert np.array_equal(ids, q3.q3_moe_topk(dev(logits), 8).cpu().numpy())
    assert np.array_equal(ids, oracle.topk_route(logits, 8))


def test_budget_round_feeds_grouped_products(q3):
    """The budget router's ids drive the grouped products; they match the oracle's
    products for the oracle's own budget routes."""
    moe = synth.make_moe(num_experts=16, k_gu=256, n_gu=96, k_dn=96, n_dn=130, tokens=8, topk=4, seed=3)
    ids_d, _ = q3.q3_moe_budget_topk(dev(moe.logits), 4, 6)
    _, ref_ids = oracle.budget_route(moe.logits, 4, 6)
    assert np.array_equal(ids_d.cpu().numpy(), ref_ids)
    st_gu = stack_experts(q3, moe.experts_gu)
    y = q3.q3_grouped_expert_gemv(st_gu, dev(moe.x), ids_d, False).cpu().numpy()
    ref, b = oracle.grouped_linear(planes(moe.experts_gu), ref_ids, moe.x, False)
    assert_close(y, ref.reshape(y.shape), b.reshape(y.shape), "budget gate/up")
    assert oracle.expert_union(ref_ids).size <= 6
