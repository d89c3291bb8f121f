"""Pins of the oracle's indexer loss: KL(target || softmax(score)) per query
row over the row's visible entries (csa_oracle_kl_from_scores, kl_loss).

The pages name the loss (a KL divergence computed by calculate_indexer_loss,
chunked over heads) but print no formula and no values, so the oracle's
reading is pinned by facts that do not come from its code: closed forms of
two-entry rows, a library routine (scipy's relative entropy of a target and
scipy's softmax), zero divergence at the softmax itself, non-negativity,
invariance to a shift of the scores, finite differences of the gradient, and
head-chunked scores giving the same loss as unchunked ones.
"""

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from synth import bf16_bits_to_f32, make_problem

NEG = -np.inf


def test_two_entry_closed_forms():
    s = np.array([[0.0, 0.0, NEG],             # equal scores, target on one entry: log 2
                  [np.log(3.0), 0.0, NEG],     # softmax (3/4, 1/4), target (1/2, 1/2): log(4/3) / 2
                  [np.log(3.0), 0.0, NEG],     # the same target unnormalised (2, 2)
                  [1.0, 2.0, NEG],             # target only on the masked entry: no mass, KL 0
                  [NEG, NEG, NEG]])            # no visible entry
    t = np.array([[1, 0, 7], [0.5, 0.5, 7], [2, 2, 7], [0, 0, 5], [1, 1, 1]], np.float32)
    kl, g = oracle.kl_from_scores(s, t, grad=True)
    np.testing.assert_allclose(kl, [np.log(2.0), 0.5 * np.log(4.0 / 3.0), 0.5 * np.log(4.0 / 3.0), 0.0, 0.0],
                               rtol=1e-14, atol=1e-15)
    # gradient softmax - p: (1/2 - 1, 1/2 - 0); (3/4 - 1/2, 1/4 - 1/2); masked entries 0
    np.testing.assert_allclose(g[0], [-0.5, 0.5, 0.0], atol=1e-15)
    np.testing.assert_allclose(g[1], [0.25, -0.25, 0.0], atol=1e-15)
    np.testing.assert_array_equal(g[3:], 0.0)


def _problem(seed, dist="gauss", segments=None, B=2, S=64, H=8, D=32, W=16, m=4):
    return make_problem(B, S, H, D, W, m, 4, dist=dist, seed=seed, segments=segments)


def _targets(P, seed, zero_frac=0.3):
    rng = np.random.default_rng(seed)
    t = rng.random((P.B, P.S, P.W)).astype(np.float32)
    t[rng.random(t.shape) < zero_frac] = 0.0
    return t


def test_matches_scipy_relative_entropy():
    """Row by row against scipy.stats.entropy(p, softmax(s)) over the visible
    entries (scipy normalises p and computes sum p log(p / q))."""
    P = _problem(3, segments="random")
    t = _targets(P, 4)
    s = oracle.scores(P)
    kl = oracle.kl_loss(P, t)
    checked = 0
    for r in range(P.B * P.S):
        vis = np.isfinite(s[r])
        tv = t.reshape(-1, P.W)[r, vis].astype(np.float64)
        if vis.sum() == 0 or tv.sum() == 0:
            assert kl[r] == 0.0
            continue
        q = scipy.special.softmax(s[r, vis].astype(np.float64))
        np.testing.assert_allclose(kl[r], scipy.stats.entropy(tv, q), rtol=1e-12, atol=1e-14)
        checked += 1
    assert checked > P.B * P.S // 2


def test_zero_at_the_softmax_and_nonnegative():
    P = _problem(5)
    s = oracle.scores(P).astype(np.float64)
    vis = np.isfinite(s)
    smax = np.max(np.where(vis, s, 0.0), axis=1, keepdims=True)
    q = np.where(vis, np.exp(np.where(vis, s, smax) - smax), 0.0)
    q = (q / np.maximum(q.sum(axis=1, keepdims=True), 1e-300)).astype(np.float32)
    kl, g = oracle.kl_from_scores(s, q, grad=True)
    assert np.all(np.abs(kl) < 1e-6)  # the target is the softmax rounded to float32
    assert np.all(np.abs(g) < 1e-6)
    kl2 = oracle.kl_loss(P, _targets(P, 6))
    assert np.all(kl2 >= -1e-12)
    assert np.any(kl2 > 1e-3)


def test_gradient_by_finite_differences_and_its_sum():
    P = _problem(7, segments="random")
    s = oracle.scores(P).astype(np.float64)
    t = _targets(P, 8).reshape(-1, P.W)
    kl, g = oracle.kl_from_scores(s, t, grad=True)
    vis = np.isfinite(s)
    np.testing.assert_array_equal(g[~vis], 0.0)
    has = (np.where(vis, t, 0).sum(axis=1) > 0)
    np.testing.assert_allclose(g.sum(axis=1)[has], 0.0, atol=1e-12)
    rng = np.random.default_rng(9)
    eps = 1e-6
    for _ in range(4):
        v = np.where(vis, rng.standard_normal(s.shape), 0.0)
        kp = oracle.kl_from_scores(np.where(vis, s + eps * v, NEG), t)
        km = oracle.kl_from_scores(np.where(vis, s - eps * v, NEG), t)
        fd = (kp - km) / (2 * eps)
        np.testing.assert_allclose(fd, np.sum(g * v, axis=1), rtol=1e-6, atol=1e-9)


def test_shift_invariance_and_masked_targets_ignored():
    P = _problem(10, segments="random")
    s = oracle.scores(P).astype(np.float64)
    t = _targets(P, 11).reshape(-1, P.W)
    vis = np.isfinite(s)
    kl, g = oracle.kl_from_scores(s, t, grad=True)
    shifted = np.where(vis, s + 7.25, NEG)
    kl2, g2 = oracle.kl_from_scores(shifted, t, grad=True)
    np.testing.assert_allclose(kl2, kl, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g2, g, atol=1e-12)
    poisoned = np.where(vis, t, np.float32(np.nan)).astype(np.float32)
    kl3, g3 = oracle.kl_from_scores(s, poisoned, grad=True)
    np.testing.assert_array_equal(kl3, kl)
    np.testing.assert_array_equal(g3, g)


def test_head_chunked_scores_give_the_same_loss():
    """On the integer grid the score is exact in float32, so summing the heads
    in chunks (the pages' head chunking, chunks of 2 and of 4 heads, numpy
    float64) gives the oracle's scores bit for bit, and the loss of either
    is the same number."""
    P = _problem(12, dist="int", H=8)
    q, k, w = (bf16_bits_to_f32(x).astype(np.float64) for x in (P.q, P.k, P.w))
    vis = np.isfinite(oracle.scores(P)).reshape(P.B, P.S, P.W)
    t = _targets(P, 13)
    ref = oracle.kl_loss(P, t)
    for chunk in (2, 4):
        sc = np.zeros((P.B, P.S, P.W))
        for h0 in range(0, P.H, chunk):
            lg = np.einsum("bhsd,bwd->bshw", q[:, h0:h0 + chunk], k)
            sc += np.einsum("bsh,bshw->bsw", w[:, :, h0:h0 + chunk], np.maximum(lg, 0.0))
        sc = np.where(vis, sc, NEG).reshape(-1, P.W)
        np.testing.assert_array_equal(sc.astype(np.float32), oracle.scores(P))
        np.testing.assert_array_equal(oracle.kl_from_scores(sc, t.reshape(-1, P.W)), ref)
