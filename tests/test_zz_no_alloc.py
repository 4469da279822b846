"""The allocation-free fused expert MLP (q3_moe_mlp_noalloc, library-owned
scratch) against the workspace entry point (q3_moe_mlp) through the C ABI: two
calls in a row, the second with a smaller round, each bitwise equal to the
workspace call and within the oracle's bound; oversized rounds rejected."""
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


def _stack(q3, layers):
    L = layers[0]
    st = q3.empty_stack(len(layers), L.n, L.k, "cuda")
    for e, layer in enumerate(layers):
        q3.q3_pack(dev(layer.codes), dev(layer.scales), dev(layer.codebook), out=st.expert(e))
    return st


def _planes(layers):
    return [(*oracle.pack(L.codes, L.scales), L.codebook, L.n, L.k) for L in layers]


def _round(q3, moe, topk, budget=None):
    st_gu, st_dn = _stack(q3, moe.experts_gu), _stack(q3, moe.experts_dn)
    x, lg = dev(moe.x), dev(moe.logits)
    if budget is None:
        ids = oracle.topk_route(moe.logits, topk)
    else:
        ids = oracle.budget_route(moe.logits, topk, budget)[1]
    idd = dev(ids)
    ws = q3.q3_moe_mlp(st_gu, st_dn, x, idd, lg).cpu().numpy()
    na = q3.q3_moe_mlp_noalloc(st_gu, st_dn, x, idd, lg).cpu().numpy()
    ref, bound = oracle.moe_mlp(_planes(moe.experts_gu), _planes(moe.experts_dn), ids, moe.logits, moe.x)
    return ws, na, ref, bound


def test_noalloc_matches_workspace_entry_point_twice(q3):
    # First the full verify round (64 experts, 8 tokens x top-8: 64 pairs,
    # I = 768, 2048 outputs), then a smaller round on other experts: the
    # scratch keeps the first call's contents, which the second must not see.
    big = synth.make_moe(seed=0)
    ws, na, ref, bound = _round(q3, big, 8)
    assert np.array_equal(na.view(np.uint32), ws.view(np.uint32))
    assert_close(na, ref, bound, "no-alloc, full round")
    small = synth.make_moe(num_experts=16, k_gu=256, n_gu=192, k_dn=96, n_dn=130, tokens=3, topk=2, seed=5)
    ws, na, ref, bound = _round(q3, small, 2, budget=3)
    assert np.array_equal(na.view(np.uint32), ws.view(np.uint32))
    assert_close(na, ref, bound, "no-alloc, smaller round")


def test_noalloc_rejects_rounds_beyond_the_scratch(q3):
    assert q3.q3_moe_mlp_noalloc_max_bytes() == 4 << 20
    # I = 8192 with 8200 outputs per pair needs more than 4 MiB at 64 pairs.
    gu = q3.empty_stack(1, 2 * 8192, 64, "cuda")
    dn = q3.empty_stack(1, 8200, 8192, "cuda")
    x = torch.zeros((8, 64), dtype=torch.int16, device="cuda")
    ids = torch.zeros((8, 8), dtype=torch.int32, device="cuda")
    lg = torch.zeros((8, 1), dtype=torch.float32, device="cuda")
    with pytest.raises(q3.Q3Error, match="UNSUPPORTED_SHAPE"):
        q3.q3_moe_mlp_noalloc(gu, dn, x, ids, lg)
