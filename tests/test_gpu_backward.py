"""GPU parity of the backward (csa_index_score_backward) against the oracle.

Integer-grid inputs with a gradient on a grid keep every product and partial
sum exact in fp32 and every gradient operand exact in bf16, so dq, dk and dw
must equal the oracle's float64 values bit for bit.  Gaussian inputs are
compared element by element against oracle.error_bounds(): the undecided
ReLU terms in full, the bf16 rounding of the gradient operand through
Hoeffding's inequality on sqrt(sum term^2), and the float32 accumulation
through the probabilistic summation bound, with each gradient's own sum
length: W for dq and dw, and for dk the 256-row chunks the kernel
accumulates (256 x the padded head count) plus the chunk count.  At the
seq-16384 shape these bounds are a few percent of |value| (the CPU pins in
test_oracle_backward.py show that they reject a dropped chunk partial and a
gradient taken from the wrong row), and 64 sampled rows and 64 entries are
checked, plus Euler's identity <q,dq> = <k,dk> = <w,dw> = <g,score>.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev_problem, to_np
from synth import make_config, make_problem

import sparse_attention_indexer_csa_amd as csa

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa.load_library()
    oracle.build(force=False)


def _grad(P, seed, grid=False):
    rng = np.random.default_rng(seed)
    if grid:
        return (rng.integers(-8, 9, size=(P.B, P.S, P.W)) * 2.0 ** -4).astype(np.float32)
    return rng.standard_normal((P.B, P.S, P.W)).astype(np.float32)


def _gpu_backward(P, g, d=None, workspace=None):
    d = d or dev_problem(P)
    gt = torch.from_numpy(g).cuda()
    return csa.score_backward(d["q"], d["k"], d["w"], gt, P.m, scale=P.scale, q_offset=d["q_offset"],
                              q_seg=d["q_seg"], k_seg=d["k_seg"], workspace=workspace)


def _assert_within(gpu, ora, bound, what):
    gpu = np.asarray(gpu, np.float64).reshape(ora.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    err = np.abs(gpu - ora)
    excess = err - bound
    worst = int(np.argmax(excess)) if excess.size else 0
    assert np.all(excess <= 0), (f"{what}: {int((excess > 0).sum())} elements outside the bound, worst flat "
                                 f"{worst}: gpu {gpu.flat[worst]} oracle {ora.flat[worst]} bound {bound.flat[worst]}")


CHUNK_ROWS = 256  # rows per partial key gradient in the kernel


def _sum_lengths(P):
    """Longest fp32 addition chain per element: (dq, dw, dk)."""
    hb = 1
    while 32 * hb < P.H:
        hb *= 2
    chunks = (P.S + CHUNK_ROWS - 1) // CHUNK_ROWS
    return P.W, P.W, min(P.S, CHUNK_ROWS) * 32 * hb + chunks


def _bounds(P, values, stats):
    """Bounds of (dq, dk, dw) from the oracle's statistics."""
    nq, nw, nk = _sum_lengths(P)
    (oq, ok, ow), (sq, sk, sw) = values, stats
    return (oracle.error_bounds(oq, sq, nq, True), oracle.error_bounds(ok, sk, nk, True),
            oracle.error_bounds(ow, sw, nw, False))


def _check(P, g, exact):
    dq, dk, dw = (to_np(t) for t in _gpu_backward(P, g))
    oq, ok, ow, sq, sk, sw = oracle.backward(P, g, stats=True)
    if exact:
        for name, a, b in (("dq", dq, oq), ("dk", dk, ok), ("dw", dw, ow)):
            b32 = b.astype(np.float32)
            assert np.array_equal(b32.astype(np.float64), b), f"{name}: oracle value not exact in fp32"
            bad = np.argwhere(a != b32)
            assert bad.size == 0, f"{P.name} {name}: {len(bad)} differ, first {bad[0]}: {a[tuple(bad[0])]} " \
                                  f"vs {b32[tuple(bad[0])]}"
    else:
        bq, bk, bw = _bounds(P, (oq, ok, ow), (sq, sk, sw))
        _assert_within(dq, oq, bq, f"{P.name} dq")
        _assert_within(dk, ok, bk, f"{P.name} dk")
        _assert_within(dw, ow, bw, f"{P.name} dw")


@pytest.mark.parametrize("shape", [
    dict(B=1, S=256, H=4, D=32, W=64, m=4),      # the tiny prefill shape
    dict(B=2, S=300, H=64, D=128, W=90, m=4),    # ragged rows, entries and chunks
    dict(B=1, S=640, H=64, D=128, W=160, m=4),   # three row chunks, two key tiles
    dict(B=1, S=130, H=100, D=64, W=130, m=1),   # padded head block, compress rate 1
    dict(B=2, S=77, H=36, D=32, W=21, m=3),
])
def test_integer_grid_exact(shape):
    P = make_problem(top_k=4, dist="int", seed=31, name=f"int{shape}", **shape)
    _check(P, _grad(P, 5, grid=True), exact=True)


@pytest.mark.parametrize("case", ["causal", "segments", "offset"])
def test_gaussian_within_bounds(case):
    kw = {"causal": {}, "segments": {"segments": "random"},
          "offset": {"q_offset": np.array([37, 1000], np.int32)}}[case]
    P = make_problem(2, 520, 64, 128, 400, 4, 4, dist="gauss", seed=41, name=f"gauss-{case}", **kw)
    _check(P, _grad(P, 6), exact=False)


def test_mid_prefill_within_bounds():
    """The mid prefill workload (S=4096, H=64, D=128, W=1024) in full."""
    P = make_config("c2")
    _check(P, _grad(P, 7), exact=False)


def test_masked_gradient_and_workspace_contents_are_ignored():
    """NaN in the gradient at masked positions and NaN in the workspace change
    nothing; two calls give the same bits."""
    P = make_problem(2, 600, 64, 128, 200, 4, 4, dist="gauss", seed=43, segments="random")
    g = _grad(P, 8)
    vis = np.isfinite(oracle.scores(P).reshape(P.B, P.S, P.W))
    d = dev_problem(P)
    ref = [to_np(t) for t in _gpu_backward(P, np.where(vis, g, 0.0).astype(np.float32), d)]
    d_ = dev_problem(P)
    need = csa.backward_workspace_size(d_["q"], d_["k"], d_["w"], P.m)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda").view(torch.uint8)
    got = [to_np(t) for t in _gpu_backward(P, np.where(vis, g, np.float32(np.nan)).astype(np.float32), d, ws)]
    again = [to_np(t) for t in _gpu_backward(P, np.where(vis, g, np.float32(np.nan)).astype(np.float32), d, ws)]
    for a, b, c in zip(ref, got, again):
        assert np.array_equal(a, b)
        assert np.array_equal(b, c)


def test_empty_shapes():
    """W=0: dq and dw are zero; S=0: dk is zero."""
    P = make_problem(1, 64, 4, 32, 0, 4, 4, dist="gauss", seed=1)
    dq, dk, dw = (to_np(t) for t in _gpu_backward(P, _grad(P, 1)))
    assert dk.size == 0 and np.all(dq == 0) and np.all(dw == 0)
    P = make_problem(2, 0, 4, 32, 16, 4, 4, dist="gauss", seed=1)
    dq, dk, dw = (to_np(t) for t in _gpu_backward(P, _grad(P, 1)))
    assert dq.size == 0 and dw.size == 0 and np.all(dk == 0)


def test_seq16384_sampled_and_euler():
    """The seq-16384 prefill (B=1, S=16384, H=64, D=128, W=4096): 64 sampled
    rows (dq, dw; chunk edges 255/256 among them) and 64 entries (dk; key
    tile edges 127/128 among them) within the oracle's bounds, and Euler's
    identity over the whole output against the GPU's own forward scores."""
    P = make_config("c3")
    g = _grad(P, 9)
    d = dev_problem(P)
    dq, dk, dw = _gpu_backward(P, g, d)
    rng = np.random.default_rng(19)
    rows = np.unique(np.concatenate([[0, 3, 4, 255, 256, 511, 512, 4095, 4096, 16127, 16128, 16383],
                                     rng.choice(16384, 52, replace=False)]))[:64]
    ents = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, 2047, 2048, 4094, 4095],
                                     rng.choice(4096, 54, replace=False)]))[:64]
    assert len(rows) == 64 and len(ents) == 64
    sq_, sw_, sk_, tq, tw, tk = oracle.backward_sample(P, g, rows, ents)
    nq, nw, nk = _sum_lengths(P)
    dq_np = to_np(dq[0][:, rows, :].permute(1, 0, 2))
    _assert_within(dq_np, sq_, oracle.error_bounds(sq_, tq, nq, True), "c3 dq rows")
    _assert_within(to_np(dw[0][rows]), sw_, oracle.error_bounds(sw_, tw, nw, False), "c3 dw rows")
    _assert_within(to_np(dk[0][ents]), sk_, oracle.error_bounds(sk_, tk, nk, True), "c3 dk entries")
    # Euler: each of <q,dq>, <k,dk>, <w,dw> equals sum over visible pairs of g * score
    sc = csa.score(d["q"], d["k"], d["w"], P.m)
    gt = torch.from_numpy(g).cuda()
    vis = torch.isfinite(sc)
    ref = torch.sum(torch.where(vis, gt.double() * torch.where(vis, sc, 0).double(), 0)).item()
    mag = torch.sum(torch.where(vis, (gt.double() * torch.where(vis, sc, 0).double()).abs(), 0)).item()
    for name, x, gx in (("q", d["q"], dq), ("k", d["k"], dk), ("w", d["w"], dw)):
        val = torch.sum(x.double() * gx.double()).item()
        assert abs(val - ref) <= 2e-3 * mag, (name, val, ref, mag)
