"""Pins of the oracle's anti-diagonal sampled block logits (the alternative
block metric of the fr page's implementation section, step 1) to things
other than its own code: the exact block log-sum-exp at stride 1, closed
forms for planted logits and constant logits, pure-Python brute force on a
tiny case, and Jensen's inequality against the pooled logit."""
import math

import numpy as np
import pytest
import scipy.special

from oracle import stem_oracle as O


def rng(seed=0):
    return np.random.default_rng(seed)


def test_stride_one_is_blockwise_logsumexp_of_causal_logits():
    # With stride 1 every causal token pair is a sample: t_ij must be the
    # log-mean-exp of the token logits of block pair (i, j) under the causal
    # mask, taken here from the full logit matrix with a library logsumexp.
    r = rng(1)
    seqlens, Hq, Hkv, d, B = [37, 70, 8], 4, 2, 8, 8
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    q = r.standard_normal((cu[-1], Hq, d))
    k = r.standard_normal((cu[-1], Hkv, d))
    t = O.antidiag_block_logits(q, k, cu, B, 1)
    cub = O.block_layout(cu, B)
    offs, _ = O.score_offsets(cub)
    for h in range(Hq):
        for s, n in enumerate(seqlens):
            qs = q[cu[s]:cu[s + 1], h]
            ks = k[cu[s]:cu[s + 1], h // 2]
            L = qs @ ks.T / math.sqrt(d)
            causal = np.tril(np.ones((n, n), bool))
            for i in range(-(-n // B)):
                for j in range(i + 1):
                    blk = L[i * B:(i + 1) * B, j * B:(j + 1) * B]
                    msk = causal[i * B:(i + 1) * B, j * B:(j + 1) * B]
                    want = scipy.special.logsumexp(blk[msk]) - math.log(msk.sum())
                    got = t[h, offs[s] + O.tri(i) + j]
                    assert abs(got - want) < 1e-12, (h, s, i, j)


@pytest.mark.parametrize("stride", [2, 4, 8])
def test_single_planted_pair(stride):
    # Every logit is 0 except the pair (x, y): logit c / sqrt(d).  If that
    # pair is on a sampled anti-diagonal (x mod stride + y mod stride =
    # stride - 1, key not after query) its sample is c / sqrt(d) / count,
    # count = stride off the diagonal tile and stride / 2 on it, and the
    # block pair's logit is log((n - 1 + e^sample) / n) with n samples
    # (gpb^2 off the diagonal block, gpb (gpb + 1) / 2 on it); every other
    # block logit is exactly 0.
    B, d, c, nblk = 16, 4, 3.0, 4
    n = B * nblk
    gpb = B // stride
    cases = [(40, 23), (45, 42), (63, 0), (17, 16), (31, 16), (5, 2), (33, 33),
             (20, 18), (47, 44), (30, 29),
             # on an anti-diagonal of a diagonal tile, key after query: never sampled
             (16, 17), (16, 19), (25, 30)]
    for x, y in cases:
        q = np.zeros((n, 1, d)); k = np.zeros((n, 1, d))
        q[x, 0, 0] = c
        k[y, 0, 0] = 1.0
        t = O.antidiag_block_logits(q, k, [0, n], B, stride)
        want = np.zeros_like(t)
        sampled = (x % stride) + (y % stride) == stride - 1 and y <= x
        if sampled:
            r_, c_ = x // stride, y // stride
            cnt = stride if r_ > c_ else stride // 2
            a = c / math.sqrt(d) / cnt
            i, j = x // B, y // B
            ne = gpb * gpb if i > j else gpb * (gpb + 1) // 2
            want[0, O.tri(i) + j] = math.log((ne - 1 + math.exp(a)) / ne)
        np.testing.assert_allclose(t, want, rtol=0, atol=1e-13, err_msg=str((x, y, sampled)))


@pytest.mark.parametrize("stride", [1, 2, 4, 8, 16])
def test_constant_logits_give_that_value_or_no_sample(stride):
    # Every token logit equals a / sqrt(d): every sample is that value, so
    # every block logit is that value, whatever the pair counts, except the
    # diagonal pair of a block that is one short group of at most stride / 2
    # tokens, whose anti-diagonal holds no causal pair: -inf there.
    B, d, a = 16, 4, 1.75
    seqlens = [1, 3, 29, 69, 16]
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    q = np.zeros((cu[-1], 2, d)); k = np.zeros((cu[-1], 1, d))
    q[:, :, 1] = a
    k[:, :, 1] = 1.0
    t = O.antidiag_block_logits(q, k, cu, B, stride)
    cub = O.block_layout(cu, B)
    offs, _ = O.score_offsets(cub)
    for s, n in enumerate(seqlens):
        for i in range(-(-n // B)):
            ni = min(B, n - i * B)
            for j in range(i + 1):
                got = t[:, offs[s] + O.tri(i) + j]
                if j == i and ni <= stride // 2:
                    assert np.all(got == -np.inf), (stride, s, i)
                else:
                    np.testing.assert_allclose(got, a / math.sqrt(d), rtol=1e-14)


def test_brute_force_loops_tiny():
    # Pure-Python loops over every (query group, key group, u) on a tiny
    # ragged case, straight from the sampling rule.
    r = rng(5)
    seqlens, B, stride, d = [13, 21], 8, 4, 3
    cu = [0, 13, 34]
    q = r.standard_normal((34, 1, d))
    k = r.standard_normal((34, 1, d))
    t = O.antidiag_block_logits(q, k, cu, B, stride)
    cub = O.block_layout(cu, B)
    offs, _ = O.score_offsets(cub)
    gpb = B // stride
    for s, n in enumerate(seqlens):
        base = cu[s]
        for i in range(-(-n // B)):
            for j in range(i + 1):
                samples = []
                for rg in range(i * gpb, (i + 1) * gpb):
                    for cg in range(j * gpb, (j + 1) * gpb):
                        vals = []
                        for u in range(stride):
                            qp = rg * stride + stride - 1 - u
                            kp = cg * stride + u
                            if qp < n and kp < n and kp <= qp:
                                vals.append(float(np.dot(q[base + qp, 0], k[base + kp, 0]))
                                            / math.sqrt(d))
                        if vals:
                            samples.append(sum(vals) / len(vals))
                want = (math.log(sum(math.exp(v) for v in samples) / len(samples))
                        if samples else -math.inf)
                got = t[0, offs[s] + O.tri(i) + j]
                assert got == pytest.approx(want, abs=1e-12), (s, i, j)


def test_jensen_against_pooled_logit():
    # At stride 1 a full off-diagonal block pair samples every token pair, and
    # the mean of its token logits is qbar_i . kbar_j / sqrt(d); log-mean-exp
    # is never below the mean (Jensen), equal only for equal logits.
    r = rng(7)
    n, B, d = 64, 16, 8
    q = r.standard_normal((n, 1, d)); k = r.standard_normal((n, 1, d))
    t = O.antidiag_block_logits(q, k, [0, n], B, 1)
    qbar = O.pool_mean(q, [0, n], B); kbar = O.pool_mean(k, [0, n], B)
    for i in range(4):
        for j in range(i):
            s_ij = float(qbar[0, i] @ kbar[0, j]) / math.sqrt(d)
            assert t[0, O.tri(i) + j] > s_ij + 1e-6


def test_metric_of_a_row_without_samples_is_zero():
    np.testing.assert_array_equal(O.metric_from_logits(np.array([-np.inf]), np.array([2.0])), [0.0])
    np.testing.assert_array_equal(
        O.metric_from_logits(np.array([-np.inf]), np.array([2.0]), "routing"), [0.0])
    assert O.metric_from_logits(np.array([-np.inf]), np.array([2.0]), "additive")[0] == -np.inf
    # a -inf entry among finite ones gets weight 0, the rest a proper softmax
    m = O.metric_from_logits(np.array([0.0, -np.inf, math.log(3.0)]), np.ones(3), "routing")
    np.testing.assert_allclose(m, [0.25, 0.0, 0.75], rtol=1e-15)


def test_prefill_with_stride_uses_sampled_metric():
    r = rng(9)
    seqlens, B, d = [100], 16, 8
    cu = [0, 100]
    q = r.standard_normal((100, 2, d)); k = r.standard_normal((100, 1, d))
    v = r.standard_normal((100, 1, d))
    ref = O.prefill(q, k, v, cu, B, 1, 2, 0.5, 4.0, score_stride=4)
    w = O.pool_vnorm(v, cu, B)
    np.testing.assert_array_equal(ref["m"], O.score_antidiag(q, k, w, cu, B, 4))
    with pytest.raises(ValueError):
        O.antidiag_block_logits(q, k, cu, B, 3)
