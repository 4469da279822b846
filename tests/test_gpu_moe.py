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


@pytest.mark.parametrize("E", [40, 64, 65, 100])
def test_topk_many_ties(q3, E):
    """Equal logits go to the lower expert, with experts in one wave or several."""
    logits = np.random.default_rng(E).integers(-2, 3, (6, E)).astype(np.float32)
    ids = q3.q3_moe_topk(dev(logits), 7).cpu().numpy()
    assert np.array_equal(ids, oracle.topk_route(logits, 7))


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


def test_grouped_more_than_64_experts(q3):
    # Past 64 experts grid row e is expert e (rows of unpicked experts exit
    # after reading the ids); up to 64, row y takes the round's y-th picked id.
    moe = synth.make_moe(num_experts=80, k_gu=256, n_gu=64, k_dn=32, n_dn=72, tokens=8, topk=4, seed=31)
    run_round(q3, moe, 4)
    ids = q3.q3_moe_topk(dev(moe.logits), 4).cpu().numpy()
    out, ref, bound = _run_mlp(q3, moe, ids)
    assert_close(out, ref, bound, "fused MLP, 80 experts")


def test_grouped_every_pair_a_different_expert(q3):
    # 64 pairs on 64 distinct experts: every grid row has work, one pair each,
    # and the rows map to the experts in increasing id order.
    moe = synth.make_moe(num_experts=64, k_gu=256, n_gu=64, k_dn=32, n_dn=72, tokens=8, topk=8, seed=32)
    ids = np.random.default_rng(32).permutation(64).astype(np.int32).reshape(8, 8)
    st_gu = stack_experts(q3, moe.experts_gu)
    st_dn = stack_experts(q3, moe.experts_dn)
    y_gu = q3.q3_grouped_expert_gemv(st_gu, dev(moe.x), dev(ids), False).cpu().numpy()
    x_dn = np.ascontiguousarray(moe.x_dn[:, :8]).reshape(64, -1)
    y_dn = q3.q3_grouped_expert_gemv(st_dn, dev(x_dn), dev(ids), True).cpu().numpy()
    ref_gu, b_gu = oracle.grouped_linear(planes(moe.experts_gu), ids, moe.x, False)
    ref_dn, b_dn = oracle.grouped_linear(planes(moe.experts_dn), ids, moe.x_dn[:, :8], True)
    assert_close(y_gu, ref_gu.reshape(64, -1), b_gu.reshape(64, -1), "gate/up, 64 distinct experts")
    assert_close(y_dn, ref_dn.reshape(64, -1), b_dn.reshape(64, -1), "down, 64 distinct experts")
    out, ref, bound = _run_mlp(q3, moe, ids)
    assert_close(out, ref, bound, "fused MLP, 64 distinct experts")


def test_grouped_only_the_highest_experts(q3):
    # Every pair on the last few experts of the stack: the round's picked ids
    # are the top of the range, served by the first grid rows.
    moe = synth.make_moe(num_experts=64, k_gu=256, n_gu=64, k_dn=32, n_dn=72, tokens=4, topk=2, seed=33)
    ids = np.array([[63, 61], [62, 63], [61, 60], [63, 60]], dtype=np.int32)
    st_gu = stack_experts(q3, moe.experts_gu)
    y_gu = q3.q3_grouped_expert_gemv(st_gu, dev(moe.x), dev(ids), False).cpu().numpy()
    ref_gu, b_gu = oracle.grouped_linear(planes(moe.experts_gu), ids, moe.x, False)
    assert_close(y_gu, ref_gu.reshape(8, -1), b_gu.reshape(8, -1), "gate/up, highest experts")
    out, ref, bound = _run_mlp(q3, moe, ids)
    assert_close(out, ref, bound, "fused MLP, highest experts")


def test_grouped_repeated_ids_take_several_slices(q3):
    # An id repeated inside a token's list gives an expert more (token, slot)
    # pairs than there are tokens, beyond the rows its block stages at once:
    # the block takes several slices.
    moe = synth.make_moe(num_experts=6, k_gu=256, n_gu=128, k_dn=64, n_dn=130, tokens=2, topk=8, seed=9)
    ids = np.array([[3, 3, 3, 3, 5, 5, 5, 5], [3, 3, 3, 3, 3, 3, 3, 3]], dtype=np.int32)
    st_gu = stack_experts(q3, moe.experts_gu)
    st_dn = stack_experts(q3, moe.experts_dn)
    y_gu = q3.q3_grouped_expert_gemv(st_gu, dev(moe.x), dev(ids), False).cpu().numpy()
    x_dn = np.ascontiguousarray(moe.x_dn[:, :8]).reshape(16, -1)
    y_dn = q3.q3_grouped_expert_gemv(st_dn, dev(x_dn), dev(ids), True).cpu().numpy()
    ref_gu, b_gu = oracle.grouped_linear(planes(moe.experts_gu), ids, moe.x, False)
    ref_dn, b_dn = oracle.grouped_linear(planes(moe.experts_dn), ids, moe.x_dn[:, :8], True)
    assert_close(y_gu, ref_gu.reshape(16, -1), b_gu.reshape(16, -1), "gate/up, repeated ids")
    assert_close(y_dn, ref_dn.reshape(16, -1), b_dn.reshape(16, -1), "down, repeated ids")
    out, ref, bound = _run_mlp(q3, moe, ids)
    assert_close(out, ref, bound, "fused MLP, repeated ids")


def test_grouped_config2_full_size(q3):
    """64 experts, gate/up 2048->1536, down 768->2048, 8 drafted tokens x top-8:
    every output row of both passes against the oracle."""
    moe = synth.make_moe(seed=0)
    u = run_round(q3, moe, 8)
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
                                             (300, 256, 8, 32), (1024, 8, 2, 3), (2, 1000, 7, 999),
                                             # the one-block-per-token router at 4, 8 and 16 token rows,
                                             # with fewer tokens than rows and absent expert lanes
                                             (3, 40, 4, 12), (5, 64, 8, 20), (12, 64, 4, 16), (16, 48, 2, 10)])
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


# Fused expert MLP (gate/up with SwiGLU, down with the routing-weight combine)
# against the oracle's fp64 composition, within 1e-3 of each output's
# first-order bound.  Random-sign rounds check every path; rounds on positive
# codebooks and activations, where the bound is within a small factor of the
# output itself, make that tolerance a sharp one; negative gate rows put the
# SwiGLU on both sides of zero.
def _mlp_planes(layers):
    return [(*oracle.pack(L.codes, L.scales), L.codebook, L.n, L.k) for L in layers]


def _sign_fixed(moe, gate_negative=False):
    """Positive codebooks and activations; optionally negative gate rows on even experts."""
    moe.x = moe.x & np.uint16(0x7FFF)
    for e, L in enumerate(moe.experts_gu):
        L.codebook = L.codebook & np.uint8(0x7F)
        if gate_negative and e % 2 == 0:
            L.codebook[: L.n // 2] |= np.uint8(0x80)
    for L in moe.experts_dn:
        L.codebook = L.codebook & np.uint8(0x7F)
    return moe


def _run_mlp(q3, moe, ids, rows=None, ws=None, logits=None):
    logits = moe.logits if logits is None else logits
    st_gu, st_dn = stack_experts(q3, moe.experts_gu), stack_experts(q3, moe.experts_dn)
    out = q3.q3_moe_mlp(st_gu, st_dn, dev(moe.x), dev(ids), dev(logits), ws).cpu().numpy()
    ref, bound = oracle.moe_mlp(_mlp_planes(moe.experts_gu), _mlp_planes(moe.experts_dn), ids, logits, moe.x,
                                rows=rows)
    if rows is not None:
        out = out[:, rows]
    return out, ref, bound


@pytest.mark.parametrize("E,k_gu,n_gu,n_dn,t,topk,sign", [
    (6, 64, 64, 40, 3, 2, "random"),          # one block column, ragged down rows
    (16, 256, 192, 130, 8, 4, "random"),      # I = 96: a half-empty gate/up block; 3 down columns
    (16, 256, 192, 130, 8, 4, "positive"),
    (8, 512, 128, 200, 5, 3, "gate_negative"),
    (4, 96, 64, 64, 1, 1, "positive"),        # one pair
    (12, 128, 256, 96, 16, 4, "positive"),    # 64 pairs
])
def test_moe_mlp_matches_oracle(q3, E, k_gu, n_gu, n_dn, t, topk, sign):
    moe = synth.make_moe(num_experts=E, k_gu=k_gu, n_gu=n_gu, k_dn=n_gu // 2, n_dn=n_dn, tokens=t, topk=topk,
                         seed=E + t + n_dn)
    if sign != "random":
        _sign_fixed(moe, gate_negative=sign == "gate_negative")
    ids = oracle.topk_route(moe.logits, topk)
    out, ref, bound = _run_mlp(q3, moe, ids)
    ratio = assert_close(out, ref, bound, f"moe mlp {sign}")
    if sign == "positive":
        assert np.all(bound <= 4 * np.abs(ref))   # the tolerance is within 0.4% of each output
    assert ratio < 1e-5


def test_moe_mlp_many_pairs_on_one_expert(q3):
    """64 tokens on one expert: four 16-token slices in gate/up, eight in down."""
    moe = _sign_fixed(synth.make_moe(num_experts=4, k_gu=128, n_gu=64, k_dn=32, n_dn=72, tokens=64, topk=1,
                                     seed=8))
    moe.logits[:, 2] += 10.0
    ids = oracle.topk_route(moe.logits, 1)
    assert np.all(ids == 2)
    out, ref, bound = _run_mlp(q3, moe, ids)
    assert_close(out, ref, bound, "one expert, 64 tokens")


def test_moe_mlp_config2_full_size(q3):
    """64 experts, gate/up 2048 -> 2 x 768, down 768 -> 2048, 8 drafted tokens x
    top-8, plain and budgeted routes: every output against the oracle."""
    moe = synth.make_moe(seed=0)
    for ids in (oracle.topk_route(moe.logits, 8), oracle.budget_route(moe.logits, 8, 16)[1]):
        out, ref, bound = _run_mlp(q3, moe, ids)
        assert_close(out, ref, bound, "config 2 fused MLP")


def test_moe_mlp_workspace_reuse_and_determinism(q3):
    """One workspace (filled with garbage first) serves consecutive rounds with
    different routes; repeated rounds are bitwise identical."""
    moe = synth.make_moe(num_experts=16, k_gu=256, n_gu=192, k_dn=96, n_dn=130, tokens=8, topk=4, seed=21)
    st_gu, st_dn = stack_experts(q3, moe.experts_gu), stack_experts(q3, moe.experts_dn)
    ws = q3.moe_mlp_workspace(st_gu, st_dn, 8, 4, "cuda")
    ws.fill_(0xFF)                  # NaN patterns everywhere
    pl_gu, pl_dn = _mlp_planes(moe.experts_gu), _mlp_planes(moe.experts_dn)
    x, logits = dev(moe.x), dev(moe.logits)
    first = None
    for rnd, budget in enumerate((None, 6, None, 4)):
        ids = oracle.topk_route(moe.logits, 4) if budget is None else oracle.budget_route(moe.logits, 4, budget)[1]
        out = q3.q3_moe_mlp(st_gu, st_dn, x, dev(ids), logits, ws).cpu().numpy()
        ref, bound = oracle.moe_mlp(pl_gu, pl_dn, ids, moe.logits, moe.x)
        assert_close(out, ref, bound, f"round {rnd}")
        if budget is None:
            if first is None:
                first = out
            else:
                assert np.array_equal(out, first)


def test_grouped_skips_out_of_range_ids(q3):
    """Pairs whose id lies outside [0, E) are skipped: their rows of y keep what
    they held, and the other pairs still match the oracle."""
    moe = synth.make_moe(num_experts=6, k_gu=64, n_gu=48, k_dn=32, n_dn=40, tokens=3, topk=2, seed=17)
    ids = oracle.topk_route(moe.logits, 2)
    bad = ids.copy()
    bad[0, 1] = -1
    bad[2, 0] = 6
    bad[2, 1] = 1 << 20
    st_gu, st_dn = stack_experts(q3, moe.experts_gu), stack_experts(q3, moe.experts_dn)
    x_dn = np.ascontiguousarray(moe.x_dn[:, :2]).reshape(6, -1)
    for st, layers, xin, xref, by_slot in [(st_gu, moe.experts_gu, moe.x, moe.x, False),
                                          (st_dn, moe.experts_dn, x_dn, moe.x_dn[:, :2], True)]:
        y = torch.full((6, st.n), 7.25, dtype=torch.float32, device="cuda")
        q3.q3_grouped_expert_gemv(st, dev(xin), dev(bad), by_slot, y)
        y = y.cpu().numpy().reshape(3, 2, -1)
        ref, b = oracle.grouped_linear(planes(layers), ids, xref, by_slot)
        for i, j in [(0, 0), (1, 0), (1, 1)]:
            assert_close(y[i, j][None], ref[i, j][None], b[i, j][None], f"pair ({i}, {j})")
        for i, j in [(0, 1), (2, 0), (2, 1)]:
            assert np.all(y[i, j] == 7.25), f"skipped pair ({i}, {j}) was written"


def test_moe_mlp_skips_out_of_range_ids(q3):
    moe = synth.make_moe(num_experts=6, k_gu=64, n_gu=64, k_dn=32, n_dn=40, tokens=3, topk=2, seed=13)
    ids = oracle.topk_route(moe.logits, 2)
    bad = ids.copy()
    bad[0, 1] = -1                  # token 0 keeps only its first expert (weight 1)
    bad[2, :] = 6                   # token 2 has none in range: its output is 0
    st_gu, st_dn = stack_experts(q3, moe.experts_gu), stack_experts(q3, moe.experts_dn)
    out = q3.q3_moe_mlp(st_gu, st_dn, dev(moe.x), dev(bad), dev(moe.logits)).cpu().numpy()
    pl_gu, pl_dn = _mlp_planes(moe.experts_gu), _mlp_planes(moe.experts_dn)
    r0, b0 = oracle.moe_mlp(pl_gu, pl_dn, ids[:1, :1], moe.logits[:1], moe.x[:1])
    r1, b1 = oracle.moe_mlp(pl_gu, pl_dn, ids[1:2], moe.logits[1:2], moe.x[1:2])
    assert_close(out[:1], r0, b0, "token 0, one slot")
    assert_close(out[1:2], r1, b1, "token 1")
    assert not out[2].any()


def test_moe_mlp_graph_replays(q3):
    """Captured in a graph, every replay (with eager work between) equals the eager result."""
    moe = synth.make_moe(num_experts=16, k_gu=256, n_gu=192, k_dn=96, n_dn=130, tokens=8, topk=4, seed=22)
    st_gu, st_dn = stack_experts(q3, moe.experts_gu), stack_experts(q3, moe.experts_dn)
    ws = q3.moe_mlp_workspace(st_gu, st_dn, 8, 4, "cuda")
    x, ids, logits = dev(moe.x), dev(oracle.topk_route(moe.logits, 4)), dev(moe.logits)
    eager = q3.q3_moe_mlp(st_gu, st_dn, x, ids, logits, ws).cpu().numpy()
    out = torch.zeros((8, 130), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        q3.q3_moe_mlp(st_gu, st_dn, x, ids, logits, ws, out)
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            q3.q3_moe_mlp(st_gu, st_dn, x, ids, logits, ws, out)
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager)
        q3.q3_moe_mlp(st_gu, st_dn, x, ids, logits, ws)      # eager work between replays
        torch.cuda.synchronize()


def _random_rounds(count=10, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        E = int(rng.integers(2, 49))
        topk = int(rng.integers(1, min(E, 8) + 1))
        t = int(rng.integers(1, 64 // topk + 1))
        n_gu = 64 * int(rng.integers(1, 9))                 # I = n_gu / 2, a multiple of 32
        k_gu = 32 * int(rng.integers(1, 65))
        n_dn = int(rng.integers(1, 400))
        budget = int(rng.integers(topk, E + 1)) if rng.random() < 0.5 else None
        out.append((E, topk, t, n_gu, k_gu, n_dn, budget))
    return out


@pytest.mark.parametrize("E,topk,t,n_gu,k_gu,n_dn,budget", _random_rounds())
def test_moe_mlp_random_rounds(q3, E, topk, t, n_gu, k_gu, n_dn, budget):
    """Seeded random rounds of the fused expert MLP (expert count, tokens,
    top-k, ragged down rows, optional expert budget).  The device router's ids
    feed the fused MLP on the device; the router is checked first (plain top-k
    exactly; a budget round exactly where the fp64 masses separate the budget
    boundary, which every round here does, see _check_budget), and the oracle
    composes the MLP over its own routes, never the GPU's."""
    moe = synth.make_moe(num_experts=E, k_gu=k_gu, n_gu=n_gu, k_dn=n_gu // 2, n_dn=n_dn, tokens=t, topk=topk,
                         seed=E * 100 + t)
    lg = dev(moe.logits)
    if budget is None:
        ids_d = q3.q3_moe_topk(lg, topk)
        ref_ids = oracle.topk_route(moe.logits, topk)
        assert np.array_equal(ids_d.cpu().numpy(), ref_ids)
    else:
        ids_d, kept = q3.q3_moe_budget_topk(lg, topk, budget)
        clear = _check_budget(moe.logits, topk, budget, ids_d.cpu().numpy(), kept.cpu().numpy())
        assert clear, "seeded round whose budget boundary is within the fp32 allowance: pick another seed"
        ref_ids = oracle.budget_route(moe.logits, topk, budget)[1]
    st_gu, st_dn = stack_experts(q3, moe.experts_gu), stack_experts(q3, moe.experts_dn)
    out = q3.q3_moe_mlp(st_gu, st_dn, dev(moe.x), ids_d, lg).cpu().numpy()
    ref, bound = oracle.moe_mlp(_mlp_planes(moe.experts_gu), _mlp_planes(moe.experts_dn), ref_ids, moe.logits, moe.x)
    assert_close(out, ref, bound, f"random round E={E} topk={topk} t={t} budget={budget}")
