"""Pins of the oracle's backward (dq, dk, dw of the indexer score).

The backward is the vector-Jacobian product of the score function: for an
upstream gradient g of the scores it returns the gradients of
L = sum over unmasked (i, j) of g[i,j] * score[i,j].  These tests tie the
oracle's closed-form loops to facts that do not come from them: finite
differences of L computed from a separate float64 formulation of the score,
Euler's theorem for positively homogeneous functions, a single-head case
that reduces to two matrix products, and the masks.
"""

import numpy as np
import pytest

import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits, make_problem


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def _mask(P):
    """[B,S,W] bool: entry visible to the row (closed form of the causal
    threshold, segments compared directly)."""
    off = np.zeros(P.B, np.int64) if P.q_offset is None else P.q_offset.astype(np.int64)
    pos = off[:, None] + np.arange(P.S)[None, :]
    thr = np.clip((pos + 1) // P.m, 0, P.W)
    vis = np.arange(P.W)[None, None, :] < thr[:, :, None]
    if P.q_seg is not None:
        vis &= P.q_seg[:, :, None] == P.k_seg[:, None, :]
    return vis


def _loss(P, q, k, w, g, vis):
    """sum over visible (i, j) of g * scale * sum_h w * ReLU(q.k), float64,
    from einsum over plain float arrays (q [B,H,S,D], k [B,W,D], w [B,S,H])."""
    logits = np.einsum("bhsd,bwd->bshw", q, k)
    score = P.scale * np.einsum("bsh,bshw->bsw", w, np.maximum(logits, 0.0))
    return float(np.sum(np.where(vis, g.astype(np.float64) * score, 0.0)))


def _problem(seed, segments=None, q_offset=None, B=2, S=40, H=8, D=32, W=12, m=4, scale=1.0):
    P = make_problem(B, S, H, D, W, m, 4, dist="gauss", seed=seed, segments=segments, scale=scale,
                     q_offset=q_offset)
    rng = np.random.default_rng(seed + 100)
    g = rng.standard_normal((B, S, W)).astype(np.float32)
    return P, g


@pytest.mark.parametrize("case", ["causal", "segments", "offset"])
def test_directional_derivatives_match_finite_differences(case):
    """<dq, v>, <dk, v>, <dw, v> equal central differences of L along random v.
    L is piecewise linear in each of q, k and w, so a small step gives the
    derivative up to float64 rounding.  Catches a wrong term, sign, index or
    factor in any of the three gradients (a transposed or shifted index moves
    the inner product with a random direction)."""
    kw = {"causal": {}, "segments": {"segments": "random", "S": 48},
          "offset": {"q_offset": np.array([5, 17], np.int32)}}[case]
    P, g = _problem(11, **kw)
    vis = _mask(P)
    q, k, w = _f64(P.q), _f64(P.k), _f64(P.w)
    dq, dk, dw = oracle.backward(P, g)
    rng = np.random.default_rng(7)
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("w", w, dw)):
        for _ in range(3):
            v = rng.standard_normal(x.shape)
            args = {"q": q, "k": k, "w": w}
            args[name] = x + eps * v
            lp = _loss(P, args["q"], args["k"], args["w"], g, vis)
            args[name] = x - eps * v
            lm = _loss(P, args["q"], args["k"], args["w"], g, vis)
            fd = (lp - lm) / (2 * eps)
            an = float(np.sum(grad * v))
            scale = float(np.sum(np.abs(grad) * np.abs(v))) + 1e-30
            assert abs(fd - an) <= 1e-6 * scale, (name, fd, an)


def test_single_element_partials():
    """A few single-element partial derivatives by finite differences: pins
    individual entries, not only inner products."""
    P, g = _problem(12)
    vis = _mask(P)
    q, k, w = _f64(P.q), _f64(P.k), _f64(P.w)
    dq, dk, dw = oracle.backward(P, g)
    rng = np.random.default_rng(3)
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("w", w, dw)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            args = {"q": q.copy(), "k": k.copy(), "w": w.copy()}
            args[name][idx] += eps
            lp = _loss(P, args["q"], args["k"], args["w"], g, vis)
            args[name][idx] -= 2 * eps
            lm = _loss(P, args["q"], args["k"], args["w"], g, vis)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7 * (1.0 + abs(grad[idx])), (name, idx, fd, grad[idx])


@pytest.mark.parametrize("scale", [1.0, 0.375])
def test_euler_homogeneity(scale):
    """The score is positively homogeneous of degree one in q, in k and in w
    separately (ReLU(c x) = c ReLU(x) for c > 0), so by Euler's theorem
    <q,dq> = <k,dk> = <w,dw> = sum of g * score over visible pairs.  The right
    side comes from the forward oracle in float64.  Catches a missing factor
    (scale, w, the indicator) or a dropped term in any gradient."""
    P, g = _problem(13, segments="random", S=48, scale=scale)
    dq, dk, dw = oracle.backward(P, g)
    s = oracle.scores(P, precision="f64").reshape(P.B, P.S, P.W)
    vis = np.isfinite(s)
    ref = float(np.sum(np.where(vis, g.astype(np.float64) * np.where(vis, s, 0.0), 0.0)))
    for name, x, grad in (("q", P.q, dq), ("k", P.k, dk), ("w", P.w, dw)):
        val = float(np.sum(_f64(x) * grad))
        assert abs(val - ref) <= 1e-12 * (1.0 + float(np.sum(np.abs(_f64(x) * grad)))), (name, val, ref)


def test_single_head_reduces_to_matmuls():
    """H=1, w=1 and positive q and k: every logit is positive, so
    dq = scale (G o V) K, dk = scale (G o V)^T Q and dw = scale rowsum(G o V o QK^T)
    with V the visibility mask (numpy matmuls, exact on the integer grid).
    Catches a swapped operand or a missing mask in either product."""
    S, D, W, m = 64, 32, 16, 4
    P = make_problem(1, S, 1, D, W, m, 4, dist="zeros", seed=0, scale=0.5)
    rng = np.random.default_rng(5)
    qv = rng.integers(1, 5, size=(1, 1, S, D)).astype(np.float32) * np.float32(2 ** -3)
    kv = rng.integers(1, 5, size=(1, W, D)).astype(np.float32) * np.float32(2 ** -3)
    P.q, P.k = f32_to_bf16_bits(qv), f32_to_bf16_bits(kv)
    P.w = f32_to_bf16_bits(np.ones((1, S, 1), np.float32))
    g = (rng.integers(-8, 9, size=(1, S, W)) * 2.0 ** -4).astype(np.float32)
    dq, dk, dw = oracle.backward(P, g)
    V = _mask(P)[0]
    G = np.where(V, g[0].astype(np.float64), 0.0)
    Q, K = qv[0, 0].astype(np.float64), kv[0].astype(np.float64)
    np.testing.assert_array_equal(dq[0, 0], 0.5 * (G @ K))
    np.testing.assert_array_equal(dk[0], 0.5 * (G.T @ Q))
    np.testing.assert_array_equal(dw[0, :, 0], 0.5 * np.sum(G * (Q @ K.T), axis=1))


def test_masked_gradient_is_ignored():
    """Values of g at masked positions (future or foreign entries) change
    nothing, not even when they are NaN: a masked score is a constant."""
    P, g = _problem(14, segments="random", S=48)
    vis = _mask(P)
    base = oracle.backward(P, np.where(vis, g, 0.0).astype(np.float32))
    poisoned = np.where(vis, g, np.float32(np.nan)).astype(np.float32)
    got = oracle.backward(P, poisoned)
    for a, b in zip(base, got):
        np.testing.assert_array_equal(a, b)


def test_statistics_cover_undecided_signs():
    """The per-element statistics are non-negative, and a logit of exactly
    zero (its ReLU derivative is undecided in float32) puts the whole term in
    the undecided mass and none of it in the decided sums."""
    P, g = _problem(15)
    dq, dk, dw, sq, sk, sw = oracle.backward(P, g, stats=True)
    for s in (sq, sk, sw):
        assert np.all(s >= 0)
    # q row i of head 0 set to zero: logit 0 for every entry, so dq[0,0,i]
    # gets no term and its undecided mass gets all of them
    i = P.S - 1
    q = _f64(P.q).copy()
    q[0, 0, i] = 0.0
    P.q = f32_to_bf16_bits(q.astype(np.float32))
    dq, dk, dw, sq, sk, sw = oracle.backward(P, g, stats=True)
    assert np.all(dq[0, 0, i] == 0.0)
    assert np.all(sq[0, 0, i, :, 0] == 0.0) and np.all(sq[0, 0, i, :, 1] == 0.0)
    nvis = int(_mask(P)[0, i].sum())
    kf = _f64(P.k)[0, :nvis]
    wv = float(_f64(P.w)[0, i, 0])
    expect = np.sum(np.abs(g[0, i, :nvis, None].astype(np.float64) * wv * kf), axis=0)
    np.testing.assert_allclose(sq[0, 0, i, :, 2], expect, rtol=1e-12)
    # the decided sums of another row are the sums of |term| and term^2
    # over its positive logits
    i2 = 20
    nv2 = int(_mask(P)[0, i2].sum())
    qh = _f64(P.q)[0, 0, i2]
    lg = _f64(P.k)[0, :nv2] @ qh
    t = (g[0, i2, :nv2].astype(np.float64) * float(_f64(P.w)[0, i2, 0]))[:, None] * _f64(P.k)[0, :nv2]
    pos = lg > 0
    np.testing.assert_allclose(sq[0, 0, i2, :, 0], np.abs(t[pos]).sum(axis=0), rtol=1e-12)
    np.testing.assert_allclose(sq[0, 0, i2, :, 1], (t[pos] ** 2).sum(axis=0), rtol=1e-12)


def test_sampled_rows_and_entries_equal_the_full_backward():
    """backward_sample (used at sizes where the full backward is too slow)
    returns the full backward's values at the chosen rows and entries."""
    P, g = _problem(16, segments="random", S=48)
    dq, dk, dw, sq, sk, sw = oracle.backward(P, g, stats=True)
    rows = [0, 5, P.S + 47, 2 * P.S - 1]
    ents = [0, 3, P.W + 11]
    xq, xw, xk, yq, yw, yk = oracle.backward_sample(P, g, rows, ents)
    for r, row in enumerate(rows):
        b, i = divmod(row, P.S)
        np.testing.assert_array_equal(xq[r], dq[b, :, i, :])
        np.testing.assert_array_equal(xw[r], dw[b, i])
        np.testing.assert_array_equal(yq[r], sq[b, :, i, :])
        np.testing.assert_array_equal(yw[r], sw[b, i])
    for e, ent in enumerate(ents):
        b, j = divmod(ent, P.W)
        np.testing.assert_array_equal(xk[e], dk[b, j])
        np.testing.assert_array_equal(yk[e], sk[b, j])


# --- the bounds at the seq-16384 shape: a float32 emulation passes, planted mistakes fail ---

CHUNK = 256  # rows per partial key gradient in the emulated implementation


def _bf16(x):
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, np.float32)))


def _emulate_dq(P, g, i, g_row):
    """dq of row i the way an fp32 kernel computes it: fp32 logits, the
    operand g [l > 0] rounded to bf16, an fp32 product with the keys, then
    scale * w.  g_row selects whose upstream gradient is used (i, or another
    row to plant a mistake)."""
    n = min((i + 1) // P.m, P.W)
    q = bf16_bits_to_f32(P.q[0, :, i, :])
    k = bf16_bits_to_f32(P.k[0, :n, :])
    lg = q @ k.T
    a = np.where(lg > 0, _bf16(g[0, g_row, :n])[None, :], np.float32(0)).astype(np.float32)
    f = (np.float32(P.scale) * bf16_bits_to_f32(P.w[0, i, :])).astype(np.float32)
    return f[:, None] * (a @ k)


def _emulate_dk(P, g, j, drop_chunk=None):
    """dk of entry j the way a chunked fp32 kernel computes it: per chunk of
    CHUNK rows the operands g w [l > 0] (fp32 product rounded to bf16)
    contracted with q in fp32, the chunk partials added in order, times the
    scale.  drop_chunk plants a lost partial.  Returns (dk, live chunks)."""
    i0 = (j + 1) * P.m - 1
    k = bf16_bits_to_f32(P.k[0, j])
    acc = np.zeros(P.D, np.float32)
    live = []
    for c in range((P.S + CHUNK - 1) // CHUNK):
        r0, r1 = max(c * CHUNK, i0), min((c + 1) * CHUNK, P.S)
        if r0 >= r1:
            continue
        live.append(c)
        Q = bf16_bits_to_f32(P.q[0, :, r0:r1, :])
        lg = Q @ k
        gw = (g[0, r0:r1, j][None, :] * bf16_bits_to_f32(P.w[0, r0:r1, :]).T).astype(np.float32)
        op = np.where(lg > 0, _bf16(gw), np.float32(0)).astype(np.float32)
        part = op.reshape(-1) @ Q.reshape(-1, P.D)
        if c != drop_chunk:
            acc = (acc + part).astype(np.float32)
    return np.float32(P.scale) * acc, live


@pytest.mark.slow
def test_bounds_at_seq16384_pass_emulation_and_catch_planted_mistakes():
    """At the seq-16384 shape (S=16384, H=64, D=128, W=4096), on sampled rows
    (255, 256, 9999) and entries (0, 127, 128, 1000), the bounds that the GPU
    backward is held to (sum lengths W for dq, CHUNK*H plus the chunk count
    for dk) admit a float32 emulation of the kernel's rounding everywhere,
    and reject most elements of two planted mistakes: dq computed with the
    next row's upstream gradient, and dk with one chunk's partial dropped."""
    from synth import make_config
    P = make_config("c3")
    g = np.random.default_rng(9).standard_normal((P.B, P.S, P.W)).astype(np.float32)
    rows, ents = [255, 256, 9999], [0, 127, 128, 1000]
    dq, dw, dk, sq, sw, sk = oracle.backward_sample(P, g, rows, ents)
    bq = oracle.error_bounds(dq, sq, P.W, True)
    bk = oracle.error_bounds(dk, sk, CHUNK * P.H + P.S // CHUNK, True)
    for r, i in enumerate(rows):
        assert np.all(np.abs(_emulate_dq(P, g, i, i) - dq[r]) <= bq[r]), f"emulated dq row {i}"
        bad = np.abs(_emulate_dq(P, g, i, i + 1) - dq[r]) > bq[r]
        assert bad.mean() > 0.9, f"swapped gradient rows: only {bad.mean():.2f} of row {i} rejected"
    for e, j in enumerate(ents):
        got, live = _emulate_dk(P, g, j)
        assert np.all(np.abs(got - dk[e]) <= bk[e]), f"emulated dk entry {j}"
        dropped, _ = _emulate_dk(P, g, j, drop_chunk=live[len(live) // 2])
        bad = np.abs(dropped - dk[e]) > bk[e]
        assert bad.mean() > 0.4, f"dropped chunk partial: only {bad.mean():.2f} of entry {j} rejected"
