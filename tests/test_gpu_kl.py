"""GPU parity of the indexer loss (csa_index_kl_loss) against the oracle.

The loss per row is KL(p || softmax(score)) over the row's visible entries
(p = the target L1-normalised there), and its gradient with respect to the
scores is softmax - p.  The kernel computes it in fp32 from its own scores:
fused into the score tiles with an online log-sum-exp (no gradient), or from
a score matrix written first (with the gradient).

Tolerances, from the arithmetic:
* the fp32 evaluation of a row: sums of at most W + 64 terms (per-lane
  chains, then lane merges) within the probabilistic summation bound
  eps = 8 sqrt(W + 64) 2^-24 of their magnitudes (oracle magnitudes:
  sum p|log p|, sum p|s|, |lse|, plus |log A| of the unnormalised target),
  the fast exp and log inside that;
* on Gaussian inputs the scores themselves may differ from the oracle's by
  ds_j = 1e-3 + 2e-3 |s_j| (the score tolerance), which moves the loss by at
  most sum_j |softmax_j - p_j| ds_j <= 2 max_j ds_j, and each softmax value
  by a factor within 2 max_j ds_j;
* on the integer grid the scores are exact (ds = 0).
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev_problem, to_np
from synth import make_config, make_problem

import sparse_attention_indexer_csa_amd as csa

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa.load_library()
    oracle.build(force=False)


def _targets(P, seed, zero_frac=0.3):
    rng = np.random.default_rng(seed)
    t = rng.random((P.B, P.S, P.W)).astype(np.float32)
    t[rng.random(t.shape) < zero_frac] = 0.0
    return t


def _gpu_kl(P, t, grad, d=None):
    d = d or dev_problem(P)
    return csa.kl_loss(d["q"], d["k"], d["w"], torch.from_numpy(t).cuda(), P.m, scale=P.scale,
                       q_offset=d["q_offset"], q_seg=d["q_seg"], k_seg=d["k_seg"], grad=grad)


def _check(P, t, exact_scores, rows=None, kl_gpu=None, grad_gpu=None):
    """Compare GPU outputs (kl [n], grad [n, W] or None) of the given rows
    with the oracle under the tolerances of the module docstring."""
    s_o = oracle.scores(P, rows).astype(np.float64)
    t_r = t.reshape(-1, P.W) if rows is None else t.reshape(-1, P.W)[rows]
    kl_o, g_o, mg = oracle.kl_from_scores(s_o, t_r, grad=True, magnitudes=True)
    vis = np.isfinite(s_o)
    A = np.where(vis, t_r.astype(np.float64), 0.0).sum(axis=1)
    eps = 8.0 * np.sqrt(P.W + 64) * U
    if exact_scores:
        ds = np.zeros(len(s_o))
    else:
        ds = np.max(np.where(vis, 1e-3 + 2e-3 * np.abs(np.where(vis, s_o, 0.0)), 0.0), axis=1)
    logA = np.abs(np.log(np.where(A > 0, A, 1.0)))
    tol = eps * (mg[:, 0] + mg[:, 1] + mg[:, 2] + logA + 1.0) + 2.0 * ds + 1e-7
    err = np.abs(kl_gpu.astype(np.float64) - kl_o)
    assert np.all(err <= tol), f"kl: worst row {int(np.argmax(err - tol))}: gpu {kl_gpu[np.argmax(err - tol)]} " \
                               f"oracle {kl_o[np.argmax(err - tol)]} tol {tol[np.argmax(err - tol)]}"
    if grad_gpu is not None:
        p = np.where(vis & (A[:, None] > 0), t_r / np.where(A > 0, A, 1.0)[:, None], 0.0)
        q = g_o + p
        rel = eps * (2.0 + mg[:, 2:3] + np.abs(np.where(vis, s_o, 0.0))) + 2.0 * ds[:, None]
        gt = rel * np.abs(q) + 4 * U * p + 1e-9
        gerr = np.abs(grad_gpu.astype(np.float64) - g_o)
        assert np.all(gerr <= gt), f"grad: {int((gerr > gt).sum())} elements outside, worst {np.max(gerr - gt)}"
        assert np.all(grad_gpu[~vis] == 0.0), "grad at masked entries must be 0"
    return kl_o


@pytest.mark.parametrize("case", [
    dict(B=1, S=256, H=4, D=32, W=64, m=4),                                  # tiny prefill shape
    dict(B=2, S=300, H=64, D=128, W=75, m=4, segments="random"),             # segments, ragged
    dict(B=2, S=200, H=100, D=64, W=50, m=4, q_offset=np.array([-9, 700], np.int32)),  # padded heads, offsets
    dict(B=1, S=150, H=16, D=32, W=150, m=1),                                # compress rate 1
])
def test_integer_grid(case):
    kw = dict(case)
    qo = kw.pop("q_offset", None)
    P = make_problem(top_k=4, dist="int", seed=17, q_offset=qo, **kw)
    t = _targets(P, 3)
    kl_f = to_np(_gpu_kl(P, t, grad=False)).reshape(-1)
    kl_g, g = (to_np(x) for x in _gpu_kl(P, t, grad=True))
    _check(P, t, True, kl_gpu=kl_f)
    _check(P, t, True, kl_gpu=kl_g.reshape(-1), grad_gpu=g.reshape(-1, P.W))


def test_mid_prefill_gaussian():
    """S=4096, H=64, D=128, W=1024 (the mid prefill workload), every row."""
    P = make_config("c2")
    t = _targets(P, 5)
    d = dev_problem(P)
    kl_f = to_np(_gpu_kl(P, t, grad=False, d=d)).reshape(-1)
    kl_g, g = (to_np(x) for x in _gpu_kl(P, t, grad=True, d=d))
    kl_o = _check(P, t, False, kl_gpu=kl_f)
    _check(P, t, False, kl_gpu=kl_g.reshape(-1), grad_gpu=g.reshape(-1, P.W))
    assert np.max(kl_o) > 0.05  # the targets are far from the softmax: a real signal


def test_long_prefill_sampled_rows():
    """The seq-16384 prefill (W=4096) fused, without a gradient, on sampled rows."""
    P = make_config("c3")
    t = _targets(P, 6)
    kl = to_np(_gpu_kl(P, t, grad=False)).reshape(-1)
    rows = np.unique(np.concatenate([[0, 3, 4, 2047, 2048, 16383], np.linspace(5, 16382, 40).astype(int)]))
    _check(P, t, False, rows=rows, kl_gpu=kl[rows])


def test_target_equal_to_softmax_and_degenerate_rows():
    """A target equal to the softmax of the oracle's scores (integer grid, so
    the GPU's scores are the same) gives KL ~ 0 and a gradient ~ 0; rows
    without visible entries or target mass give exactly 0."""
    P = make_problem(1, 64, 16, 32, 16, 4, 4, dist="int", seed=23)
    s = oracle.scores(P).astype(np.float64)
    vis = np.isfinite(s)
    smax = np.max(np.where(vis, s, 0.0), axis=1, keepdims=True)
    e = np.where(vis, np.exp(np.where(vis, s, smax) - smax), 0.0)
    t = (e / np.maximum(e.sum(axis=1, keepdims=True), 1e-300)).astype(np.float32).reshape(P.B, P.S, P.W)
    t[0, 40] = 0.0                       # a row with no target mass
    kl, g = (to_np(x) for x in _gpu_kl(P, t, grad=True))
    kl_f = to_np(_gpu_kl(P, t, grad=False))
    assert np.all(kl[0, :3] == 0.0) and np.all(g[0, :3] == 0.0)   # rows 0..2 see no entry
    assert kl[0, 40] == 0.0 and np.all(g[0, 40] == 0.0) and kl_f[0, 40] == 0.0
    assert np.max(np.abs(kl)) < 1e-5 and np.max(np.abs(g)) < 1e-5
    _check(P, t, True, kl_gpu=kl_f.reshape(-1))
