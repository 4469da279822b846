"""GPU parity of the two-bit draft head (Hibana page, "Model surgery" / "Two-bit
draft head"): 2-bit packing bit-exact; 2-bit scores and FP8 rescoring within
|y - y_ref| <= 1e-3 * sum_k |x_k w_k|; the shortlist bit-exact against the
oracle on host-drawn fp32 scores (ties included).  Where fp32 scores decide
the list and the decision inside the pipeline, the GPU's choices must follow
its own scores exactly (plain numpy ranking, same rule) and be valid against
the oracle's fp64 scores within the rounding allowance; the oracle only ever
sees host inputs."""
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


def pack_head(q3, head):
    w2 = q3.q3_pack2(dev(head.codes), dev(head.scales), dev(head.codebook))
    h8 = q3.Mxfp8Head(head.n, head.k, dev(head.e8), dev(head.s8))
    return w2, h8


@pytest.mark.parametrize("n,k", [(1024, 1024), (37, 96), (5, 32), (64, 160), (100, 4096), (3, 8224)])
def test_pack2_bit_exact(q3, n, k):
    head, _ = synth.make_head(n, k, 1, seed=n + k)
    w2, _ = pack_head(q3, head)
    cp, sp = oracle.pack2(head.codes, head.scales)
    assert np.array_equal(w2.code_plane.cpu().numpy(), cp)
    assert np.array_equal(w2.scale_plane.cpu().numpy(), sp)
    codes, scales = q3.q3_unpack2(w2)
    assert np.array_equal(codes.cpu().numpy(), head.codes & 3)
    assert np.array_equal(scales.cpu().numpy(), head.scales)


def test_pack2_worked_example(q3):
    # K = 32, one group: codebook 1, 2, -1, 0.5, scale 2^-1, code k % 4, x = 1 -> 10
    codes = torch.tensor((np.arange(32) % 4).astype(np.uint8)[None, :]).cuda()
    scales = torch.tensor([[126]], dtype=torch.uint8).cuda()
    cb = torch.tensor([[0x38, 0x40, 0xB8, 0x30]], dtype=torch.uint8).cuda()
    w2 = q3.q3_pack2(codes, scales, cb)
    x = torch.full((1, 32), 0x3F80, dtype=torch.int16).cuda()
    assert q3.q3_head2_scores(w2, x).cpu().numpy()[0, 0] == 10.0


@pytest.mark.parametrize("n,k,m", [(1024, 1024, 1), (333, 1056, 3), (4096, 4096, 1), (2000, 4096, 16),
                                   (17, 32, 5), (513, 2048, 8)])
def test_head2_scores_parity(q3, n, k, m):
    head, x = synth.make_head(n, k, m, seed=3 * n + k + m)
    w2, _ = pack_head(q3, head)
    y = q3.q3_head2_scores(w2, dev(x)).cpu().numpy()
    cp, sp = oracle.pack2(head.codes, head.scales)
    y_ref, bound = oracle.linear2(cp, sp, head.codebook, n, k, x)
    assert_close(y, y_ref, bound, f"head2 n={n} k={k} m={m}")


def _check_list(ids, vals, scores, size):
    """ids/vals are exactly the oracle's shortlist of these (host-drawn) fp32 scores."""
    want = oracle.shortlist(scores, size)
    assert np.array_equal(ids, want)
    assert np.array_equal(vals, np.take_along_axis(scores, want.astype(np.int64), axis=1))


@pytest.mark.parametrize("m,n,size,ties", [(1, 151936, 16, False), (3, 1000, 16, True), (2, 17, 16, True),
                                           (1, 16, 16, False), (4, 70000, 5, True), (1, 1024, 1, False),
                                           # up to 4 rows per lane of the first pass (four-entry lists), then more
                                           # (full lists), and more than one load batch per lane
                                           (1, 262144, 16, True), (2, 262145, 16, True), (1, 300000, 16, False),
                                           (1, 1100000, 16, True)])
def test_shortlist_exact(q3, m, n, size, ties):
    rng = np.random.default_rng(n + size)
    if ties:
        scores = rng.integers(-4, 5, (m, n)).astype(np.float32)   # many equal scores
    else:
        scores = rng.standard_normal((m, n)).astype(np.float32)
    ids, vals = q3.q3_shortlist(torch.from_numpy(scores).cuda(), size)
    _check_list(ids.cpu().numpy(), vals.cpu().numpy(), scores, size)


def test_shortlist_strided_rows(q3):
    rng = np.random.default_rng(7)
    big = rng.standard_normal((3, 5000)).astype(np.float32)
    t = torch.from_numpy(big).cuda()[:, :4321]
    ids, vals = q3.q3_shortlist(t, 16)
    _check_list(ids.cpu().numpy(), vals.cpu().numpy(), big[:, :4321], 16)


def ranked(scores, size):
    """Plain numpy ranking (score desc, row asc): used to check that the GPU's
    list and decision agree with the GPU's own scores."""
    out = []
    for row in np.asarray(scores, dtype=np.float64):
        out.append(np.lexsort((np.arange(row.size), -row))[:size])
    return np.array(out)


def oracle_rescore_all(head, x, block=8192):
    """Oracle FP8 scores and bounds of every row for every query (host inputs only)."""
    m = x.shape[0]
    y = np.empty((m, head.n))
    b = np.empty((m, head.n))
    for r0 in range(0, head.n, block):
        r = np.arange(r0, min(head.n, r0 + block))
        ids = np.broadcast_to(np.arange(r.size), (m, r.size))
        y[:, r], b[:, r] = oracle.rescore(head.e8[r], head.s8[r], x, ids)
    return y, b


def check_decision(ids, y8, best, y_ref_all, b_ref_all):
    """best is the top of the GPU's own scores of its list, and no listed row
    beats it in the oracle's scores by more than the rounding allowance."""
    m = ids.shape[0]
    for i in range(m):
        order = sorted(range(ids.shape[1]), key=lambda t: (-float(y8[i, t]), int(ids[i, t])))
        assert best[i] == ids[i, order[0]]
        lo = y_ref_all[i, best[i]] + 1e-3 * b_ref_all[i, best[i]]
        hi = np.max(y_ref_all[i, ids[i]] - 1e-3 * b_ref_all[i, ids[i]])
        assert lo >= hi


@pytest.mark.parametrize("n,k,m,size", [(200, 4096, 1, 16), (300, 1056, 3, 7), (40, 32, 2, 16),
                                        (64, 4128, 2, 5), (90, 9216, 1, 16)])   # second, partial 4096-wide slice
def test_rescore_parity_and_decision(q3, n, k, m, size):
    head, x = synth.make_head(n, k, m, seed=n * k + m)
    _, h8 = pack_head(q3, head)
    rng = np.random.default_rng(size)
    ids = rng.integers(0, n, (m, size)).astype(np.int32)
    ids[0, 0] = ids[0, -1]          # a row listed twice
    y, best = q3.q3_rescore_fp8(h8, dev(x), torch.from_numpy(ids).cuda())
    y, best = y.cpu().numpy(), best.cpu().numpy()
    y_ref, bound = oracle.rescore(head.e8, head.s8, x, ids)
    assert_close(y, y_ref, bound, "rescore")
    y_all, b_all = oracle_rescore_all(head, x)
    check_decision(ids, y, best, y_all, b_all)


def test_rescore_out_of_range_ids_score_zero(q3):
    head, x = synth.make_head(64, 256, 1, seed=9)
    _, h8 = pack_head(q3, head)
    ids = np.array([[3, -1, 64, 5]], dtype=np.int32)
    y, _ = q3.q3_rescore_fp8(h8, dev(x), torch.from_numpy(ids).cuda())
    y = y.cpu().numpy()
    assert y[0, 1] == 0 and y[0, 2] == 0
    y_ref, bound = oracle.rescore(head.e8, head.s8, x, ids[:, [0, 3]])
    assert_close(y[:, [0, 3]], y_ref, bound, "rescore in-range ids")


def check_list_valid(ids, s2_gpu, s64, b64):
    """The list is the top of the GPU's own scores (exact ranking rule), and
    against the oracle's fp64 scores no unlisted row beats a listed one by more
    than the two scores' rounding allowance."""
    assert np.array_equal(ids, ranked(s2_gpu, ids.shape[1]))
    for i in range(ids.shape[0]):
        listed = np.zeros(s64.shape[1], bool)
        listed[ids[i]] = True
        assert np.min(s64[i, listed] + 1e-3 * b64[i, listed]) >= np.max(s64[i, ~listed] - 1e-3 * b64[i, ~listed])


@pytest.mark.parametrize("n,k,m", [(5000, 1024, 1), (3000, 512, 4)])
def test_draft_head_end_to_end(q3, n, k, m):
    head, x = synth.make_head(n, k, m, seed=n + m)
    w2, h8 = pack_head(q3, head)
    xd = dev(x)
    ids, y8, best = q3.q3_draft_head(w2, h8, xd, 16)
    ids, y8, best = ids.cpu().numpy(), y8.cpu().numpy(), best.cpu().numpy()
    s2 = q3.q3_head2_scores(w2, xd).cpu().numpy()
    cp, sp = oracle.pack2(head.codes, head.scales)
    s64, b64 = oracle.linear2(cp, sp, head.codebook, n, k, x)
    assert_close(s2, s64, b64, "2-bit scores")
    check_list_valid(ids, s2, s64, b64)
    y_all, b_all = oracle_rescore_all(head, x)
    assert_close(y8, np.take_along_axis(y_all, ids.astype(np.int64), 1),
                 np.take_along_axis(b_all, ids.astype(np.int64), 1), "draft head rescore")
    check_decision(ids, y8, best, y_all, b_all)


def test_draft_head_full_size(q3):
    """Vocabulary-sized head (K=4096, N=151936), one query: the 2-bit scores of
    every row against the oracle's fp64 scores, the list valid against those
    fp64 scores on every row (and exactly the ranking of the GPU's own scores),
    FP8 scores of the listed rows and the decision."""
    n, k = 151936, 4096
    head, x = synth.make_head(n, k, 1, seed=0)
    w2, h8 = pack_head(q3, head)
    xd = dev(x)
    ids, y8, best = q3.q3_draft_head(w2, h8, xd, 16)
    ids, y8, best = ids.cpu().numpy(), y8.cpu().numpy(), best.cpu().numpy()
    s2 = q3.q3_head2_scores(w2, xd).cpu().numpy()
    cp, sp = oracle.pack2(head.codes, head.scales)
    s64, b64 = oracle.linear2(cp, sp, head.codebook, n, k, x)
    assert_close(s2, s64, b64, "full-size 2-bit scores")
    check_list_valid(ids, s2, s64, b64)
    y_all, b_all = oracle_rescore_all(head, x)
    assert_close(y8, y_all[:, ids[0]], b_all[:, ids[0]], "full-size rescore")
    check_decision(ids, y8, best, y_all, b_all)
