"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names the plausible oracle mistake it would catch.  The oracle is
the definition of the indexer score written as loops; these tests tie it to
closed forms, to a library routine in a special case, to brute force and to
invariants of the method (head permutation, causality, packed documents,
decode = last prefill row, power-of-two scaling).
"""

import json
import os

import numpy as np
import pytest

import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits, make_config, make_problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _visible_counts(S, m, W, offset=0):
    # Closed form of the causal threshold: entry j is visible once all m
    # tokens of its block are at or before the row's position.
    return np.clip((np.arange(S) + offset + 1) // m, 0, W)


def _rank1_problem(S, H, D, W, m, top_k, a, c, w_rows, offset=None):
    """q[h,i] = a[h,i] e0, k[j] = c[j] e0, w[i,h] given."""
    P = make_problem(1, S, H, D, W, m, top_k, dist="zeros", seed=0)
    q = np.zeros((1, H, S, D), np.float32)
    q[0, :, :, 0] = a
    k = np.zeros((1, W, D), np.float32)
    k[0, :, 0] = c
    P.q, P.k = _bf16(q), _bf16(k)
    P.w = _bf16(np.asarray(w_rows, np.float32).reshape(1, S, H))
    if offset is not None:
        P.q_offset = np.array([offset], np.int32)
    return P


# --- golden: hand-derived worked example ------------------------------------

def test_golden_hand_derived_example():
    """Catches any error in the score formula, the mask or the tie rule on a case
    derived by hand (tests/golden/closed_form_tiny.json)."""
    g = json.load(open(os.path.join(GOLDEN, "closed_form_tiny.json")))
    sh = g["shape"]
    S, H, D, W, m, k = sh["S"], sh["H"], sh["D"], sh["W"], sh["m"], sh["top_k"]
    a = np.tile(np.asarray(g["inputs"]["q_head_coeff"], np.float32)[:, None], (1, S))
    w = np.tile(np.asarray(g["inputs"]["w_row"], np.float32)[None, :], (S, 1))
    P = _rank1_problem(S, H, D, W, m, k, a, g["inputs"]["k_coeff"], w)
    s, idx = oracle.select(P)
    expect_idx = np.zeros((S, k), np.int32)
    for rng_s, row in g["expected_idx"].items():
        lo, hi = (int(x) for x in rng_s.split("-")) if "-" in rng_s else (int(rng_s), int(rng_s))
        expect_idx[lo:hi + 1] = row
    np.testing.assert_array_equal(idx, expect_idx)
    es = np.asarray(g["entry_scores"], np.float32)
    for i in range(S):
        n = min(W, (i + 1) // m)
        np.testing.assert_array_equal(s[i, :n], es[:n])
        assert np.all(np.isneginf(s[i, n:]))


# --- closed forms -------------------------------------------------------------

@pytest.mark.parametrize("offset", [None, 5])
def test_all_ties_closed_form(offset):
    """q = 0 makes every visible score 0.  The selection must then be the first
    min(k, visible) entries in index order: catches a causal off-by-one, a wrong
    tie direction, wrong padding or a wrong use of q_offset."""
    S, H, D, W, m, k = 64, 3, 32, 16, 4, 6
    P = make_problem(1, S, H, D, W, m, k, dist="gauss", seed=11)
    P.q = np.zeros_like(P.q)
    if offset is not None:
        P.q_offset = np.array([offset], np.int32)
    s, idx = oracle.select(P)
    nvis = _visible_counts(S, m, W, offset or 0)
    # spot values of the threshold, written out: with m=4 and no offset,
    # rows 0..2 see nothing, row 3 sees entry 0, row 7 sees entries 0..1.
    if offset is None:
        assert list(nvis[[0, 2, 3, 6, 7, 11, 63]]) == [0, 0, 1, 1, 2, 3, 16]
    for i in range(S):
        n = nvis[i]
        assert np.all(s[i, :n] == 0.0) and np.all(np.signbit(s[i, :n]) == 0)
        assert np.all(np.isneginf(s[i, n:]))
        expect = list(range(min(k, n))) + [-1] * (k - min(k, n))
        assert list(idx[i]) == expect


def test_rank1_increasing_closed_form():
    """k[j] = (j+1)/64 e0, q = a e0 (a>0), w>0: score = a c_j sum(w) exactly and
    strictly increasing in j, so idx = thr-1, thr-2, ...: catches a reversed
    order, a dropped head or a wrong scale."""
    S, H, D, W, m, k = 256, 4, 32, 64, 4, 16
    a = np.full((H, S), 0.5, np.float32)
    c = (np.arange(W, dtype=np.float32) + 1) / 64.0
    wr = np.tile(np.array([0.25, 0.5, 1.0, 2.0], np.float32), (S, 1))
    P = _rank1_problem(S, H, D, W, m, k, a, c, wr)
    s, idx = oracle.select(P)
    nvis = _visible_counts(S, m, W)
    for i in range(S):
        n = nvis[i]
        np.testing.assert_array_equal(s[i, :n], (0.5 * c[:n] * 3.75).astype(np.float32))
        expect = [n - 1 - t for t in range(min(k, n))] + [-1] * (k - min(k, n))
        assert list(idx[i]) == expect


def test_relu_and_weight_sign_closed_form():
    """Rank-1 logits a[h,i] c[j] of both signs and weights of both signs.
    For c_j > 0 only heads with a > 0 pass the ReLU, for c_j < 0 only heads with
    a < 0, so score = c_j * sum_{h: a c_j > 0} w[i,h] a[h,i] (all dyadic, exact).
    Catches a missing ReLU, ReLU after weighting, and w or q index transposition."""
    S, H, D, W, m, k = 32, 4, 32, 8, 4, 8
    rng = np.random.default_rng(7)
    a = rng.choice(np.array([-1.0, -0.5, 0.5, 1.0, 2.0], np.float32), size=(H, S))
    c = np.array([0.25, -0.5, 0.75, -0.125, 1.0, -1.5, 0.375, -0.25], np.float32)
    wr = rng.choice(np.array([-1.0, -0.25, 0.5, 0.75], np.float32), size=(S, H))
    P = _rank1_problem(S, H, D, W, m, k, a, c, wr)
    s = oracle.scores(P)
    nvis = _visible_counts(S, m, W)
    for i in range(S):
        pos = sum(float(wr[i, h]) * float(a[h, i]) for h in range(H) if a[h, i] > 0)
        neg = sum(float(wr[i, h]) * float(a[h, i]) for h in range(H) if a[h, i] < 0)
        for j in range(W):
            if j >= nvis[i]:
                assert np.isneginf(s[i, j])
                continue
            expect = float(c[j]) * (pos if c[j] > 0 else neg)
            assert s[i, j] == np.float32(expect) + np.float32(0.0), (i, j)


# --- library special case ------------------------------------------------------

@pytest.mark.parametrize("D", [32, 128])
def test_single_head_is_relu_matmul(D):
    """H=1, w=1: the score is ReLU(Q K^T) masked, and the selection is a stable
    descending sort (numpy matmul and lexsort).  Integer-grid inputs keep every
    sum exact.  Catches dropped or misindexed terms of the dot product and any
    error in the selection order."""
    S, W, m, k = 96, 24, 4, 10
    P = make_problem(1, S, 1, D, W, m, k, dist="int", seed=3)
    P.w = _bf16(np.ones((1, S, 1), np.float32))
    s, idx = oracle.select(P)
    qf = bf16_bits_to_f32(P.q[0, 0]).astype(np.float64)  # [S,D]
    kf = bf16_bits_to_f32(P.k[0]).astype(np.float64)  # [W,D]
    ref = np.maximum(qf @ kf.T, 0.0)
    nvis = _visible_counts(S, m, W)
    for i in range(S):
        n = nvis[i]
        np.testing.assert_array_equal(s[i, :n].astype(np.float64), ref[i, :n])
        j = np.arange(n)
        order = np.lexsort((j, -ref[i, :n]))[:k]
        expect = list(order) + [-1] * (k - len(order))
        assert list(idx[i]) == expect


# --- brute force -----------------------------------------------------------------

def test_topk_brute_force_membership_and_order():
    """Selection checked pair by pair: every chosen entry beats every valid
    entry left out, chosen entries are in (score desc, j asc) order, no masked
    entry is chosen, no duplicates, count = min(k, valid).  Scores drawn from a
    tiny set so that ties are common."""
    rng = np.random.default_rng(5)
    rows, W, k = 40, 23, 7
    sc = rng.choice(np.array([-1.0, 0.0, 0.5, 0.5, 2.0], np.float32), size=(rows, W))
    sc[rng.random((rows, W)) < 0.3] = -np.inf
    sc[0, :] = -np.inf
    sc[1, 3] = -0.0
    idx = oracle.topk(sc, k)

    def beats(i, a, b):
        return sc[i, a] > sc[i, b] or (sc[i, a] == sc[i, b] and a < b)

    for i in range(rows):
        valid = [j for j in range(W) if np.isfinite(sc[i, j])]
        chosen = [j for j in idx[i] if j >= 0]
        assert len(chosen) == min(k, len(valid))
        assert len(set(chosen)) == len(chosen)
        assert all(j in valid for j in chosen)
        assert all(x == -1 for x in idx[i][len(chosen):])
        for a_, b_ in zip(chosen, chosen[1:]):
            assert beats(i, a_, b_)
        for a_ in chosen:
            for b_ in valid:
                if b_ not in chosen:
                    assert beats(i, a_, b_)


def test_topk_negative_zero_ties_with_zero():
    """-0 and +0 compare equal, so they tie and the lower index goes first."""
    sc = np.array([[-np.inf, 0.0, -0.0, 1.0, -0.0]], np.float32)
    assert list(oracle.topk(sc, 4)[0]) == [3, 1, 2, 4]


# --- invariants ------------------------------------------------------------------

@pytest.mark.parametrize("dist", ["int", "gauss"])
def test_head_permutation_invariance(dist):
    """Permuting heads of q together with w leaves scores unchanged (bitwise on
    the integer grid, to rounding on Gaussian): catches a head-index mix-up
    between q and w or a dropped head."""
    P = make_problem(1, 64, 8, 32, 16, 4, 5, dist=dist, seed=9)
    perm = np.random.default_rng(1).permutation(8)
    Q = make_problem(1, 64, 8, 32, 16, 4, 5, dist=dist, seed=9)
    Q.q = np.ascontiguousarray(P.q[:, perm])
    Q.w = np.ascontiguousarray(P.w[:, :, perm])
    s1, i1 = oracle.select(P)
    s2, i2 = oracle.select(Q)
    if dist == "int":
        np.testing.assert_array_equal(s1, s2)
        np.testing.assert_array_equal(i1, i2)
    else:
        fin = np.isfinite(s1)
        assert np.array_equal(fin, np.isfinite(s2))
        np.testing.assert_allclose(s1[fin], s2[fin], rtol=1e-5, atol=1e-6)


def test_batch_rows_are_independent():
    """Each batch row of a B=3 problem equals the same data run alone: catches
    batch-stride errors in q, k, w, q_offset or segment ids."""
    P = make_problem(3, 40, 4, 32, 10, 4, 4, dist="int", seed=21, segments="random",
                     q_offset=np.array([0, 3, 17], np.int32))
    s, idx = oracle.select(P)
    for b in range(3):
        Q = make_problem(1, 40, 4, 32, 10, 4, 4, dist="int", seed=21)
        Q.q, Q.k, Q.w = P.q[b:b + 1].copy(), P.k[b:b + 1].copy(), P.w[b:b + 1].copy()
        Q.q_offset = P.q_offset[b:b + 1].copy()
        Q.q_seg, Q.k_seg = P.q_seg[b:b + 1].copy(), P.k_seg[b:b + 1].copy()
        s1, i1 = oracle.select(Q)
        np.testing.assert_array_equal(s1, s[b * 40:(b + 1) * 40])
        np.testing.assert_array_equal(i1, idx[b * 40:(b + 1) * 40])


def test_future_and_foreign_entries_are_never_read():
    """Poisoning keys a row may not see (future entries, other documents) with
    huge values leaves that row's scores and selection unchanged."""
    P = make_problem(1, 128, 4, 32, 32, 4, 8, dist="gauss", seed=4, segments="random")
    s, idx = oracle.select(P)
    J0 = 20
    Q = make_problem(1, 128, 4, 32, 32, 4, 8, dist="gauss", seed=4, segments="random")
    kk = bf16_bits_to_f32(Q.k).copy()
    kk[0, J0:] = 8.0
    Q.k = _bf16(kk)
    s2, i2 = oracle.select(Q)
    rows = np.where(_visible_counts(128, 4, 32) <= J0)[0]
    np.testing.assert_array_equal(s[rows], s2[rows])
    np.testing.assert_array_equal(idx[rows], i2[rows])
    # foreign-segment poisoning: row i keeps its output when every entry of
    # another document is poisoned
    for i in (60, 100, 127):
        R = make_problem(1, 128, 4, 32, 32, 4, 8, dist="gauss", seed=4, segments="random")
        kk = bf16_bits_to_f32(R.k).copy()
        kk[0, R.k_seg[0] != R.q_seg[0, i]] = 8.0
        R.k = _bf16(kk)
        s3, i3 = oracle.select(R, rows=[i])
        np.testing.assert_array_equal(s3[0], s[i])
        np.testing.assert_array_equal(i3[0], idx[i])


def test_masked_entries_never_selected_and_counts():
    """Invariants of the selection on a packed-segment problem: chosen entries
    are valid, distinct, count = min(k, n_valid), ordered by score."""
    P = make_problem(2, 200, 8, 64, 50, 4, 12, dist="gauss", seed=8, segments="random")
    s, idx = oracle.select(P)
    v = oracle.valid(P)
    assert np.array_equal(v, np.isfinite(s))
    for r in range(P.rows):
        chosen = idx[r][idx[r] >= 0]
        assert len(chosen) == min(P.top_k, int(v[r].sum()))
        assert len(set(chosen.tolist())) == len(chosen)
        assert v[r, chosen].all()
        sc = s[r, chosen]
        assert np.all(sc[:-1] >= sc[1:])


@pytest.mark.parametrize("dist", ["int", "gauss"])
def test_decode_row_equals_last_prefill_row(dist):
    """A one-row decode call at position S-1 over the same cache equals row S-1
    of the prefill (bitwise): catches a q_offset error."""
    S, H, D, W, m, k = 128, 4, 64, 32, 4, 9
    P = make_problem(2, S, H, D, W, m, k, dist=dist, seed=13)
    s, idx = oracle.select(P)
    Q = make_problem(2, 1, H, D, W, m, k, dist=dist, seed=13)
    Q.q = np.ascontiguousarray(P.q[:, :, S - 1:S])
    Q.w = np.ascontiguousarray(P.w[:, S - 1:S])
    Q.k = P.k.copy()
    Q.q_offset = np.array([S - 1, S - 1], np.int32)
    s1, i1 = oracle.select(Q)
    for b in range(2):
        np.testing.assert_array_equal(s1[b], s[b * S + S - 1])
        np.testing.assert_array_equal(i1[b], idx[b * S + S - 1])


def test_chunked_prefill_equals_unchunked():
    """Rows s0..S-1 computed as a chunk with q_offset = s0 equal those rows of
    the whole prefill (the chunked == unchunked idea of the head-chunking PR)."""
    S, H, D, W, m, k, s0 = 120, 4, 32, 30, 4, 6, 48
    P = make_problem(1, S, H, D, W, m, k, dist="gauss", seed=14)
    s, idx = oracle.select(P)
    Q = make_problem(1, S - s0, H, D, W, m, k, dist="gauss", seed=14)
    Q.q = np.ascontiguousarray(P.q[:, :, s0:])
    Q.w = np.ascontiguousarray(P.w[:, s0:])
    Q.k = P.k.copy()
    Q.q_offset = np.array([s0], np.int32)
    s1, i1 = oracle.select(Q)
    np.testing.assert_array_equal(s1, s[s0:])
    np.testing.assert_array_equal(i1, idx[s0:])


def test_packed_documents_equal_unpacked():
    """With documents aligned to the compress rate, each document's rows in the
    packed problem equal the document run alone, indices shifted by start/m
    (the packed == unpacked selection idea of the selection-flags PR)."""
    S, H, D, m, k = 256, 4, 32, 4, 6
    W = S // m
    P = make_problem(2, S, H, D, W, m, k, dist="gauss", seed=15, segments="aligned")
    s, idx = oracle.select(P)
    checked = 0
    for b in range(2):
        seg = P.q_seg[b]
        for d in np.unique(seg):
            toks = np.where(seg == d)[0]
            st, en = int(toks[0]), int(toks[-1]) + 1
            assert st % m == 0 and en % m == 0
            L = en - st
            Q = make_problem(1, L, H, D, L // m, m, k, dist="gauss", seed=0)
            Q.q = np.ascontiguousarray(P.q[b:b + 1, :, st:en])
            Q.w = np.ascontiguousarray(P.w[b:b + 1, st:en])
            Q.k = np.ascontiguousarray(P.k[b:b + 1, st // m:en // m])
            s1, i1 = oracle.select(Q)
            rows = b * S + np.arange(st, en)
            np.testing.assert_array_equal(s1, s[rows][:, st // m:en // m])
            shifted = np.where(i1 >= 0, i1 + st // m, -1)
            np.testing.assert_array_equal(shifted, idx[rows])
            checked += 1
    assert checked >= 2


def test_power_of_two_scaling_is_exact():
    """scale = 2^e, or w multiplied by 2^e, multiplies every score by exactly
    2^e and leaves the selection unchanged: catches a misplaced scale."""
    P = make_problem(1, 64, 8, 32, 16, 4, 5, dist="gauss", seed=16)
    s, idx = oracle.select(P)
    P2 = make_problem(1, 64, 8, 32, 16, 4, 5, dist="gauss", seed=16, scale=0.25)
    s2, i2 = oracle.select(P2)
    fin = np.isfinite(s)
    np.testing.assert_array_equal(s2[fin], s[fin] * np.float32(0.25))
    np.testing.assert_array_equal(i2, idx)
    P3 = make_problem(1, 64, 8, 32, 16, 4, 5, dist="gauss", seed=16)
    P3.w = _bf16(bf16_bits_to_f32(P3.w) * 2.0)
    s3, i3 = oracle.select(P3)
    np.testing.assert_array_equal(s3[fin], s[fin] * np.float32(2.0))
    np.testing.assert_array_equal(i3, idx)


# --- rounding of the oracle itself -------------------------------------------------

def test_integer_grid_is_exact_in_fp32():
    """On the integer grid every partial sum is exact in fp32: the fp32 oracle
    equals its float64 twin bit for bit (c1 shape and a c2-like shape)."""
    P = make_config("c1")
    np.testing.assert_array_equal(oracle.scores(P).astype(np.float64), oracle.scores(P, precision="f64"))
    Q = make_problem(1, 512, 64, 128, 128, 4, 32, dist="int", seed=22)
    rows = np.arange(200, 512, 7)
    np.testing.assert_array_equal(oracle.scores(Q, rows).astype(np.float64),
                                  oracle.scores(Q, rows, precision="f64"))


def test_fp32_oracle_error_is_far_below_tolerance():
    """On Gaussian inputs the fp32 oracle stays within 1e-6 of its float64 twin,
    three orders below the parity tolerance (1e-3 abs / 2e-3 rel)."""
    Q = make_problem(1, 1024, 64, 128, 256, 4, 64, dist="gauss", seed=2)
    rows = np.arange(0, 1024, 5)
    s32 = oracle.scores(Q, rows).astype(np.float64)
    s64 = oracle.scores(Q, rows, precision="f64")
    fin = np.isfinite(s64)
    assert np.array_equal(fin, np.isfinite(s32))
    err = np.abs(s32[fin] - s64[fin])
    assert err.max() < 1e-6, err.max()


# --- stored regression fixture -----------------------------------------------------

def test_c1_regression_fixture():
    """The oracle still reproduces the fixture written by
    tests/golden/make_golden.py (which calls only the oracle)."""
    g = json.load(open(os.path.join(GOLDEN, "c1_oracle.json")))
    P = make_config("c1")
    s, idx = oracle.select(P)
    np.testing.assert_array_equal(idx, np.asarray(g["idx"], np.int32))
    for r, row in zip(g["score_rows"], g["scores_hex"]):
        got = [float(x).hex() for x in s[r]]
        assert got == row
