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
