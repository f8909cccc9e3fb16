"""Pins of the CPU oracle to things other than itself: closed forms, brute
force on tiny inputs, library routines and the budget tables derived by hand
from the decay rule.  None of these tests needs a GPU."""
import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import stem_oracle as O
from tests._golden import pages_parameters
from block_sparse_causal_amd import synthetic as syn


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- pooling


def test_pool_identical_rows_give_that_row():
    r = rng(1)
    B, d = 8, 16
    row = np.round(r.standard_normal((1, 2, d)) * 64) / 64   # dyadic: sums are exact
    x = np.repeat(row, 3 * B, axis=0)                 # 3 blocks of identical rows
    out = O.pool_mean(x, [0, 3 * B], B)
    for j in range(3):
        np.testing.assert_array_equal(out[:, j, :], row[0])


def test_pool_vnorm_of_axis_rows_is_mean_abs():
    # V rows c_t * e_1 have ||v_t|| = |c_t|; the block value is mean |c_t|.
    B, d = 4, 8
    c = np.array([3.0, -4.0, 0.5, -0.5, 2.0, 2.0, -2.0, 6.0])
    v = np.zeros((8, 1, d))
    v[:, 0, 0] = c
    w = O.pool_vnorm(v, [0, 8], B)
    assert w.shape == (1, 2)
    assert w[0, 0] == pytest.approx((3 + 4 + 0.5 + 0.5) / 4, abs=0, rel=1e-15)
    assert w[0, 1] == pytest.approx((2 + 2 + 2 + 6) / 4, rel=1e-15)
    wm = O.pool_vnorm(v, [0, 8], B, mode="max")
    assert list(wm[0]) == [4.0, 6.0]


def test_pool_brute_force_loops_with_ragged_tail_and_varlen():
    r = rng(2)
    B, H, d = 4, 3, 5
    seqlens = [10, 0, 7, 4]                      # ragged tails and an empty sequence
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    x = r.standard_normal((int(cu[-1]), H, d))
    got = O.pool_mean(x, cu, B)
    gw = O.pool_vnorm(x, cu, B)
    # brute force: walk tokens one at a time
    want, wantw = [], []
    for s, n in enumerate(seqlens):
        nb = (n + B - 1) // B
        for jl in range(nb):
            toks = [int(cu[s]) + t for t in range(jl * B, min(n, (jl + 1) * B))]
            acc = [[0.0] * d for _ in range(H)]
            accw = [0.0] * H
            for t in toks:
                for h in range(H):
                    sq = 0.0
                    for e in range(d):
                        acc[h][e] += x[t, h, e]
                        sq += x[t, h, e] ** 2
                    accw[h] += math.sqrt(sq)
            want.append([[a / len(toks) for a in acc[h]] for h in range(H)])
            wantw.append([a / len(toks) for a in accw])
    want = np.array(want).transpose(1, 0, 2)
    wantw = np.array(wantw).T
    assert got.shape == (H, 3 + 0 + 2 + 1, d)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(gw, wantw, rtol=1e-13, atol=1e-13)


def test_pool_is_linear():
    r = rng(3)
    B = 16
    x = r.standard_normal((64, 2, 8))
    y = r.standard_normal((64, 2, 8))
    a, b = 1.5, -0.25
    np.testing.assert_allclose(O.pool_mean(a * x + b * y, [0, 64], B),
                               a * O.pool_mean(x, [0, 64], B) + b * O.pool_mean(y, [0, 64], B),
                               rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- metric


def test_score_hand_computed_row():
    # d = 4 so the scale is 1/2.  qbar_1 = 2 ln3 e1, kbar_0 = 0, kbar_1 = e1
    # -> logits [0, ln 3] -> softmax [1/4, 3/4]; w = [2, 4] -> m = [1/2, 3].
    qbar = np.zeros((1, 2, 4)); qbar[0, 1, 0] = 2 * math.log(3.0)
    kbar = np.zeros((1, 2, 4)); kbar[0, 1, 0] = 1.0
    w = np.array([[2.0, 4.0]])
    m = O.score(qbar, kbar, w, np.array([0, 2]), 4)
    # packed rows: row 0 = [m00], row 1 = [m10, m11]
    assert m.shape == (1, 3)
    assert m[0, 0] == pytest.approx(2.0, rel=1e-15)          # a row of one block: p = 1
    assert m[0, 1] == pytest.approx(0.5, rel=1e-14)
    assert m[0, 2] == pytest.approx(3.0, rel=1e-14)


def test_score_zero_query_gives_w_over_row_length():
    r = rng(4)
    nb, d = 9, 8
    qbar = np.zeros((2, nb, d))
    kbar = r.standard_normal((1, nb, d))
    w = r.uniform(0.5, 3.0, (1, nb))
    cub = np.array([0, nb])
    m = O.score(qbar, kbar, w, cub, d)
    for h in range(2):
        for i in range(nb):
            np.testing.assert_allclose(O.score_row(m, cub, h, 0, i), w[0, :i + 1] / (i + 1),
                                       rtol=1e-14)


def test_score_unit_w_is_library_softmax_and_gqa_uses_group_head():
    r = rng(5)
    nb, d, Hq, Hkv = 7, 16, 4, 2
    qbar = r.standard_normal((Hq, nb, d))
    kbar = r.standard_normal((Hkv, nb, d))
    w = np.ones((Hkv, nb))
    cub = np.array([0, nb])
    m = O.score(qbar, kbar, w, cub, d)
    for h in range(Hq):
        g = h // 2                                  # contiguous groups of 2
        for i in range(nb):
            lg = np.array([np.dot(qbar[h, i], kbar[g, j]) for j in range(i + 1)]) / 4.0
            np.testing.assert_allclose(O.score_row(m, cub, h, 0, i),
                                       scipy.special.softmax(lg), rtol=1e-13)


def test_score_rows_are_per_sequence():
    # two sequences: the second one's row i must only see its own blocks
    r = rng(6)
    d = 8
    qbar = r.standard_normal((1, 5, d))
    kbar = r.standard_normal((1, 5, d))
    w = r.uniform(1, 2, (1, 5))
    cub = np.array([0, 2, 5])
    m = O.score(qbar, kbar, w, cub, d)
    assert m.shape == (1, 3 + 6)
    sub = O.score(qbar[:, 2:], kbar[:, 2:], w[:, 2:], np.array([0, 3]), d)
    np.testing.assert_array_equal(m[:, 3:], sub)


def test_metric_orders_like_additive_oam_with_half_beta():
    # log m_ij = s_ij + log w_j - log Z_i: same order as s + (1/2) log ||V||^2
    # (the pages' additive metric) when log w^2 > 0.
    r = rng(7)
    nb, d = 40, 32
    qbar = r.standard_normal((1, nb, d))
    kbar = r.standard_normal((1, nb, d))
    w = r.uniform(1.5, 20.0, (1, nb))
    cub = np.array([0, nb])
    m = O.score(qbar, kbar, w, cub, d)
    i = nb - 1
    s = kbar[0] @ qbar[0, i] / math.sqrt(d)
    additive = s + 0.5 * np.maximum(0.0, np.log(w[0] ** 2))
    np.testing.assert_array_equal(np.argsort(-O.score_row(m, cub, 0, 0, i), kind="stable"),
                                  np.argsort(-additive, kind="stable"))


def test_additive_metric_hand_computed_row():
    # d = 4 (scale 1/2), qbar_2 = 2 e1, kbar = [0, e1, -e1] -> s = [0, 1, -1];
    # w = [e, 1/2, 0]: log w^2 = [2, -2 ln 2, -inf] -> bonus beta*[2, 0, 0].
    qbar = np.zeros((1, 3, 4)); qbar[0, 2, 0] = 2.0
    kbar = np.zeros((1, 3, 4)); kbar[0, 1, 0] = 1.0; kbar[0, 2, 0] = -1.0
    w = np.array([[math.e, 0.5, 0.0]])
    m = O.score(qbar, kbar, w, np.array([0, 3]), 4, metric="additive", beta=0.75)
    row = O.score_row(m, np.array([0, 3]), 0, 0, 2)
    np.testing.assert_allclose(row, [0.75 * 2.0, 1.0, -1.0], rtol=1e-15, atol=1e-15)
    # beta = 0 leaves the scaled logits alone
    m0 = O.score(qbar, kbar, w, np.array([0, 3]), 4, metric="additive", beta=0.0)
    np.testing.assert_allclose(O.score_row(m0, np.array([0, 3]), 0, 0, 2), [0.0, 1.0, -1.0],
                               atol=1e-15)


def test_additive_metric_rows_are_not_normalised():
    # the additive form has no softmax: adding a constant to every logit of a
    # row (a query component along a direction all kbar share) shifts the row
    r = rng(71)
    nb, d = 6, 8
    kbar = r.standard_normal((1, nb, d)); kbar[0, :, 0] = 1.0
    qbar = r.standard_normal((1, nb, d)); qbar[0, :, 0] = 0.0
    q2 = qbar.copy(); q2[0, :, 0] = 3.0
    w = r.uniform(0.5, 4.0, (1, nb))
    cub = np.array([0, nb])
    a = O.score(qbar, kbar, w, cub, d, metric="additive", beta=0.3)
    b = O.score(q2, kbar, w, cub, d, metric="additive", beta=0.3)
    np.testing.assert_allclose(b - a, 3.0 / math.sqrt(d), rtol=1e-12)


def test_routing_metric_is_softmax_and_ignores_w():
    r = rng(72)
    nb, d = 9, 16
    qbar = r.standard_normal((2, nb, d))
    kbar = r.standard_normal((1, nb, d))
    w = r.uniform(0.1, 9.0, (1, nb))
    cub = np.array([0, nb])
    m = O.score(qbar, kbar, w, cub, d, metric="routing")
    for h in range(2):
        for i in range(nb):
            lg = kbar[0, :i + 1] @ qbar[h, i] / 4.0
            np.testing.assert_allclose(O.score_row(m, cub, h, 0, i),
                                       scipy.special.softmax(lg), rtol=1e-13)
    # and equals the output-aware metric with every w = 1
    m1 = O.score(qbar, kbar, np.ones_like(w), cub, d)
    np.testing.assert_allclose(m, m1, rtol=1e-15)


def test_unknown_metric_is_rejected():
    with pytest.raises(ValueError):
        O.score(np.zeros((1, 1, 4)), np.zeros((1, 1, 4)), np.ones((1, 1)), np.array([0, 1]), 4,
                metric="oam")


# ---------------------------------------------------------------- budget


# Executed blocks per head, summed over query blocks, derived from the decay
# rule by hand (see the per-workload notes below) and independently of this
# oracle.
BUDGET_TOTALS = {
    "single-head-1k-fp32": 58,
    "llama3-8b-32k-b64": 5922,
    "llama3-8b-128k-b128": 19285,
    "qwen2.5-7b-64k-b64": 20864,
    "llama3-8b-varlen-120k-b64": 28774,
}


@pytest.mark.parametrize("name", list(syn.WORKLOADS))
def test_budget_totals(name):
    w = syn.WORKLOADS[name]
    cub = O.block_layout(w.cu_seqlens, w.block)
    bud = O.budgets_for(cub, w.sink_blocks, w.k_min, w.rho0, w.tau)
    assert int(bud.sum()) == BUDGET_TOTALS[name]


def test_budget_closed_forms():
    # single head 1k: S=1, k_min=2, rho0=1, tau=4: ceil((i+1)e^{-i/4}) <= 2 for
    # all i, so k_dyn = 2 and k_i = min(i+1, 4) -> [1,2,3,4,4,...]
    b = O.budget(16, 1, 2, 1.0, 4.0)
    assert list(b) == [1, 2, 3] + [4] * 13
    # headline: 0.3 (i+1) e^{-i/128} peaks near i+1 = 128 at 14.2 < 16, so
    # k_dyn = 16 and k_i = min(i+1, 19)
    b = O.budget(1024, 2, 16, 0.3, 128.0)
    assert list(b) == [min(i + 1, 19) for i in range(1024)]
    # rho0 = 0 is the uniform budget k_min
    b = O.budget(50, 3, 5, 0.0, 10.0)
    assert list(b) == [min(i + 1, 9) if i >= 3 else i + 1 for i in range(50)]
    # first rows below the sinks keep every causal block
    b = O.budget(6, 4, 1, 0.5, 2.0)
    assert list(b[:4]) == [1, 2, 3, 4]
    # 32k llama: 0.5 (i+1) e^{-i/64} peaks at 0.5*64*e^{-63/64} = 11.96 -> 12
    b = O.budget(512, 2, 8, 0.5, 64.0)
    assert b.max() == 2 + 1 + 12 and b[-1] == 2 + 1 + 8


def test_budget_linear_endpoints():
    # mu of the pages' ablation (tests/golden/pages_parameters.txt): 0.7
    mu = pages_parameters()["mu"]
    assert mu == 0.7
    b = O.budget_linear(101, 2, 0, 20, mu)
    assert b[2] == 3                               # row 2 has only 3 causal blocks
    assert b[50] == 2 + 1 + math.ceil(20 * 0.5 + 14 * 0.5)
    assert b[100] == 2 + 1 + 14                    # k_end = mu * k_start
    # once the causal cap stops binding the dynamic part never rises
    kd = b[25:] - 3
    assert (np.diff(kd) <= 0).all() and kd[0] <= 20 and kd[-1] == 14


def test_budget_linear_special_cases():
    # mu = 1: uniform k_start (rounded up); k_min floors it
    b = O.budget_linear(64, 1, 0, 5.5, 1.0)
    assert list(b) == [1] + [min(i + 1, 1 + 1 + 6) for i in range(1, 64)]
    b = O.budget_linear(64, 1, 9, 5.5, 1.0)
    assert list(b) == [1] + [min(i + 1, 1 + 1 + 9) for i in range(1, 64)]
    # mu = 0 decays to nothing but the floor at the last block
    b = O.budget_linear(33, 0, 2, 16, 0.0)
    assert b[32] == 1 + 2 and b[16] == 1 + 8
    # one block: f = 0
    assert list(O.budget_linear(1, 0, 0, 3, 0.5)) == [1]
    # the per-sequence table restarts at every sequence
    cub = np.array([0, 10, 10, 40])
    t = O.budgets_for(cub, 2, 1, 0.0, 1.0, mode="linear", k_start=8, mu=0.25)
    np.testing.assert_array_equal(t, np.concatenate([O.budget_linear(10, 2, 1, 8, 0.25),
                                                     O.budget_linear(30, 2, 1, 8, 0.25)]))


def test_budget_linear_fraction_hand_table():
    # nb = 5, S = 1, k_min = 0, k_start = 0.5, mu = 0.5: f = i/4, share
    # r = 0.5(1 - f) + 0.25 f; k_dyn = ceil(r (i+1)): i=1 -> ceil(0.875) = 1,
    # i=2 -> ceil(1.125) = 2, i=3 -> ceil(1.25) = 2, i=4 -> ceil(1.25) = 2;
    # k_i = min(i+1, 1 + 1 + k_dyn)
    assert list(O.budget_linear_fraction(5, 1, 0, 0.5, 0.5)) == [1, 2, 3, 4, 4]


def test_budget_linear_fraction_special_cases():
    # the whole causal row at every block: dense causal attention
    assert list(O.budget_linear_fraction(40, 2, 0, 1.0, 1.0)) == list(range(1, 41))
    # a zero share leaves the floor k_min
    assert list(O.budget_linear_fraction(30, 1, 3, 0.0, 0.5)) == \
        [1] + [min(i + 1, 1 + 1 + 3) for i in range(1, 30)]
    # mu = 1: a constant share, ceil(r (i+1)) blocks, here r = 1/4
    b = O.budget_linear_fraction(64, 0, 0, 0.25, 1.0)
    assert list(b) == [min(i + 1, 1 + math.ceil(0.25 * (i + 1))) for i in range(64)]
    # mu = 0: the share reaches zero at the last block
    b = O.budget_linear_fraction(33, 0, 2, 0.5, 0.0)
    assert b[32] == 1 + 2 and b[16] == 1 + math.ceil(0.25 * 17)
    # one block: f = 0
    assert list(O.budget_linear_fraction(1, 0, 0, 0.3, 0.5)) == [1]
    # the per-sequence table restarts at every sequence
    cub = np.array([0, 7, 7, 40])
    t = O.budgets_for(cub, 2, 1, 0.0, 1.0, mode="linear_fraction", k_start=0.4, mu=0.7)
    np.testing.assert_array_equal(
        t, np.concatenate([O.budget_linear_fraction(7, 2, 1, 0.4, 0.7),
                           O.budget_linear_fraction(33, 2, 1, 0.4, 0.7)]))


def test_additive_metric_beta_default_is_the_pages_value():
    import inspect
    from block_sparse_causal_amd import synthetic as syn
    beta = pages_parameters()["beta"]
    for fn in (O.score, O.score_row_values, O.metric_from_logits, O.score_antidiag, O.prefill):
        assert inspect.signature(fn).parameters["beta"].default == beta, fn.__name__
    assert syn.custom([64], 1, 1, 64, "bf16", 64).beta == beta


# ---------------------------------------------------------------- selection


def brute_select(m_row, i, k_i, S):
    forced = set(range(min(S, i + 1))) | {i}
    cand = list(range(S, i))
    take = max(0, k_i - len(forced))
    take = min(take, len(cand))

    def better(a, b):  # a strictly before b in the ranking
        va, vb = m_row[a], m_row[b]
        if np.isnan(va):
            return False if not np.isnan(vb) else a < b
        if np.isnan(vb):
            return True
        return va > vb or (va == vb and a < b)

    hits = []
    for sub in itertools.combinations(cand, take):
        rest = [c for c in cand if c not in sub]
        if all(better(a, b) for a in sub for b in rest):
            hits.append(sub)
    assert len(hits) == 1
    return sorted(forced | set(hits[0]))


@pytest.mark.parametrize("seed", range(6))
def test_select_matches_brute_force(seed):
    r = rng(100 + seed)
    for i in range(0, 12):
        row = r.uniform(0, 1, i + 1)
        if seed % 2:                                  # plenty of ties
            row = np.round(row * 4) / 4
        if seed == 5 and i > 3:
            row[2] = np.nan
        for S in (0, 1, 2, 3):
            for k_i in range(1, i + 2):
                if k_i < min(S, i + 1) + (1 if i >= S else 0):
                    continue
                got = O.select_row(row, i, k_i, S)
                assert list(got) == brute_select(row, i, k_i, S)


def test_select_invariants_and_scale_invariance():
    w = syn.custom([1000, 300], 4, 2, 32, "f32", 16, sink_blocks=2, k_min=3, rho0=0.6, tau=5.0)
    x = syn.generate(w)
    res = O.prefill(x.q, x.k, x.v, w.cu_seqlens, w.block, w.sink_blocks, w.k_min, w.rho0, w.tau)
    cub, idx, cnt, bud = res["cu_blocks"], res["idx"], res["count"], res["budget"]
    for h in range(4):
        for s in range(2):
            for i in range(int(cub[s + 1] - cub[s])):
                b = int(cub[s]) + i
                sel = idx[h, b, :cnt[h, b]]
                assert cnt[h, b] == bud[b]
                assert np.all(np.diff(sel) > 0) and sel[0] >= 0 and sel[-1] == i
                assert set(range(min(2, i + 1))) <= set(sel.tolist())
                assert np.all(idx[h, b, cnt[h, b]:] == -1)
    # scaling the block magnitudes by c > 0 scales m by c and keeps the selection
    m2 = res["m"] * 7.5
    idx2, cnt2 = O.select(m2, cub, bud, 2)
    np.testing.assert_array_equal(idx2, idx)


def test_select_all_ties_picks_smallest_index():
    row = np.ones(20)
    assert list(O.select_row(row, 19, 2 + 1 + 5, 2)) == [0, 1, 2, 3, 4, 5, 6, 19]
    row = np.zeros(20); row[-0] = -0.0
    row[5] = -0.0
    assert list(O.select_row(row, 19, 4, 2)) == [0, 1, 2, 19]


# ---------------------------------------------------------------- attention


def torch_masked_attention(q, k, v, allowed):
    """Library reference: scaled_dot_product_attention in float64 on the CPU
    with an explicit boolean mask [Tq, Tk]."""
    qt = torch.from_numpy(q.astype(np.float64)).transpose(0, 1)[None]   # [1, H, T, d]
    kt = torch.from_numpy(k.astype(np.float64)).transpose(0, 1)[None]
    vt = torch.from_numpy(v.astype(np.float64)).transpose(0, 1)[None]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(allowed)[None, None])
    return o[0].transpose(0, 1).numpy()


def test_full_budget_equals_dense_and_library():
    w = syn.custom([96, 70], 4, 2, 16, "f32", 16, sink_blocks=1, k_min=1000, rho0=0.0)
    x = syn.generate(w)
    res = O.prefill(x.q, x.k, x.v, w.cu_seqlens, w.block, w.sink_blocks, w.k_min, w.rho0, w.tau)
    od, lsed = O.dense_causal_attn(x.q, x.k, x.v, w.cu_seqlens)
    np.testing.assert_allclose(res["o"], od, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(res["lse"], lsed, rtol=1e-12, atol=1e-12)
    cu = w.cu_seqlens
    for s in range(2):
        a, e = int(cu[s]), int(cu[s + 1])
        qq = x.q[a:e]
        kk = np.repeat(x.k[a:e], 2, axis=1)
        vv = np.repeat(x.v[a:e], 2, axis=1)
        ref = torch_masked_attention(qq, kk, vv, np.tril(np.ones((e - a, e - a), bool)))
        np.testing.assert_allclose(res["o"][a:e], ref, rtol=1e-11, atol=1e-11)


def test_sparse_equals_library_with_block_mask():
    w = syn.custom([200, 77], 2, 1, 16, "f32", 16, sink_blocks=2, k_min=2, rho0=0.3, tau=3.0)
    x = syn.generate(w)
    res = O.prefill(x.q, x.k, x.v, w.cu_seqlens, w.block, w.sink_blocks, w.k_min, w.rho0, w.tau)
    cu, cub, B = w.cu_seqlens, res["cu_blocks"], w.block
    for s in range(2):
        a, e = int(cu[s]), int(cu[s + 1])
        n = e - a
        for h in range(2):
            allowed = np.zeros((n, n), bool)
            for i in range(int(cub[s + 1] - cub[s])):
                b = int(cub[s]) + i
                for j in res["idx"][h, b, :res["count"][h, b]]:
                    allowed[i * B:(i + 1) * B, j * B:(j + 1) * B] = True
            allowed &= np.tril(np.ones((n, n), bool))
            ref = torch_masked_attention(x.q[a:e, h:h + 1], x.k[a:e], x.v[a:e], allowed)
            np.testing.assert_allclose(res["o"][a:e, h], ref[:, 0], rtol=1e-11, atol=1e-11)
            # LSE against the library logsumexp of the masked logits
            lg = torch.from_numpy(x.q[a:e, h].astype(np.float64) @ x.k[a:e, 0].astype(np.float64).T / 4.0)
            lg = lg.masked_fill(~torch.from_numpy(allowed), -math.inf)
            np.testing.assert_allclose(res["lse"][h, a:e], torch.logsumexp(lg, 1).numpy(), rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    B, d = 8, 4
    T = 40
    r = rng(9)
    q = r.standard_normal((T, 1, d))
    k = r.standard_normal((T, 1, d))
    cu = [0, T]
    nb = T // B
    idx = np.full((1, nb, 3), -1, np.int32)
    cnt = np.zeros((1, nb), np.int32)
    for i in range(nb):
        sel = sorted({0, i, max(0, i - 2)})
        idx[0, i, :len(sel)] = sel
        cnt[0, i] = len(sel)
    # constant V rows -> output is that row
    vc = np.tile(np.array([1.5, -2.0, 0.25, 3.0]), (T, 1, 1))
    o, _ = O.sparse_attn(q, k, vc, idx, cnt, cu, B)
    np.testing.assert_allclose(o[:, 0], vc[:, 0], rtol=1e-14)
    # Q = 0 -> o_t = mean of the allowed v_s
    v = r.standard_normal((T, 1, d))
    o, lse = O.sparse_attn(np.zeros_like(q), k, v, idx, cnt, cu, B)
    for t in range(T):
        i = t // B
        allowed = [s for j in idx[0, i, :cnt[0, i]] for s in range(j * B, j * B + B) if s <= t]
        np.testing.assert_allclose(o[t, 0], v[allowed, 0].mean(axis=0), rtol=1e-13, atol=1e-14)
        assert lse[0, t] == pytest.approx(math.log(len(allowed)), rel=1e-14)
    # the first token of a sequence sees only itself -> o = v_0
    o, _ = O.sparse_attn(q, k, v, idx, cnt, cu, B)
    np.testing.assert_array_equal(o[0, 0], v[0, 0])


# ---------------------------------------------------------------- generator


def test_generator_bf16_rounding_matches_torch():
    r = rng(11)
    x = (r.standard_normal(100000) * np.exp(r.uniform(-20, 20, 100000))).astype(np.float32)
    ours = syn.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_generator_is_deterministic_and_shaped():
    w = syn.custom([64, 33], 4, 2, 16, "bf16", 16)
    a = syn.generate(w)
    b = syn.generate(w)
    np.testing.assert_array_equal(a.q_bits, b.q_bits)
    assert a.q.shape == (97, 4, 16) and a.k.shape == (97, 2, 16)
    np.testing.assert_array_equal(syn.bf16_bits_to_f32(a.v_bits), a.v)
    # K of the first 4 tokens of each sequence is scaled by 3 (before bf16 rounding)
    assert np.abs(a.k[64:68]).mean() > 2 * np.abs(a.k[68:]).mean()
