"""Helpers of the GPU parity tests: move a synth.Problem to the device, call
the library through its binding, and compare with the oracle under the
parity rules.

Parity rules (the indexer's stated precision: bf16 inputs, fp32 accumulation):
* integer-grid inputs: every partial sum is exact in fp32, so scores and
  indices must match the oracle bit for bit;
* Gaussian inputs: scores within 2e-3 relative / 1e-3 absolute
  (|gpu - oracle| <= 1e-3 + 2e-3 |oracle|), masked entries exactly -inf on both
  sides; top-k sets equal in size, and any entry in one set but not the other
  has an oracle score within that tolerance of the oracle's k-th score.
"""

from __future__ import annotations

import numpy as np
import torch

import sparse_attention_indexer_csa_amd as csa

RTOL = 2e-3
ATOL = 1e-3


def dev_problem(P, device="cuda", layout="head_major"):
    """Device tensors of a Problem.  layout="seq_major" stores q as [B,S,H,D]
    and returns the permuted [B,H,S,D] view (D still contiguous)."""
    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    if layout == "head_major":
        q = bf16(P.q)
    elif layout == "seq_major":
        q = bf16(np.ascontiguousarray(P.q.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
    else:
        raise ValueError(layout)
    d = dict(q=q, k=bf16(P.k), w=bf16(P.w))

    def i32(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)

    d["q_offset"] = i32(P.q_offset)
    d["q_seg"] = i32(P.q_seg)
    d["k_seg"] = i32(P.k_seg)
    return d


def gpu_select(P, plan="auto", return_scores=False, dev=None, top_k=None):
    d = dev or dev_problem(P)
    return csa.select(d["q"], d["k"], d["w"], top_k or P.top_k, P.m, scale=P.scale, q_offset=d["q_offset"],
                      q_seg=d["q_seg"], k_seg=d["k_seg"], plan=plan, return_scores=return_scores)


def gpu_score(P, plan="auto", dev=None):
    d = dev or dev_problem(P)
    return csa.score(d["q"], d["k"], d["w"], P.m, scale=P.scale, q_offset=d["q_offset"], q_seg=d["q_seg"],
                     k_seg=d["k_seg"], plan=plan)


def to_np(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def assert_scores_close(gpu, ora, exact=False, what=""):
    gpu = np.asarray(gpu, np.float32).reshape(ora.shape)
    mask_o = np.isneginf(ora)
    mask_g = np.isneginf(gpu)
    assert np.array_equal(mask_o, mask_g), f"{what}: masks differ at {np.argwhere(mask_o != mask_g)[:5]}"
    fin = ~mask_o
    assert np.all(np.isfinite(gpu[fin])), f"{what}: non-finite GPU scores"
    if exact:
        bad = np.argwhere(gpu.view(np.uint32) != ora.view(np.uint32))
        assert bad.size == 0, f"{what}: {len(bad)} scores differ bitwise, first {bad[:5]} " \
                              f"gpu={gpu[tuple(bad[0])]} oracle={ora[tuple(bad[0])]}"
    else:
        err = np.abs(gpu[fin].astype(np.float64) - ora[fin])
        lim = ATOL + RTOL * np.abs(ora[fin].astype(np.float64))
        worst = int(np.argmax(err - lim)) if err.size else 0
        assert np.all(err <= lim), f"{what}: max excess {(err - lim).max()} at flat {worst}"


def assert_topk_match(gpu_idx, ora_idx, ora_scores, exact=False, what=""):
    """gpu_idx, ora_idx: [rows, k]; ora_scores: [rows, W] oracle fp32 scores."""
    g = np.asarray(gpu_idx).reshape(ora_idx.shape)
    if exact:
        bad = np.argwhere(g != ora_idx)
        assert bad.size == 0, f"{what}: {len(bad)} indices differ, first row {bad[0][0]}: " \
                              f"gpu={g[bad[0][0]][:8]} oracle={ora_idx[bad[0][0]][:8]}"
        return
    k = ora_idx.shape[1]
    W = ora_scores.shape[1]
    for r in range(g.shape[0]):
        gs, os_ = g[r], ora_idx[r]
        ng, no = int((gs >= 0).sum()), int((os_ >= 0).sum())
        assert ng == no, f"{what}: row {r}: {ng} selected vs oracle {no}"
        assert np.all(gs[ng:] == -1), f"{what}: row {r}: padding not at the end"
        sel = gs[:ng]
        assert np.all((sel >= 0) & (sel < W)), f"{what}: row {r}: index out of range"
        assert len(set(sel.tolist())) == ng, f"{what}: row {r}: duplicate index"
        assert np.all(np.isfinite(ora_scores[r, sel])), f"{what}: row {r}: masked entry selected"
        diff = set(sel.tolist()) ^ set(os_[:no].tolist())
        if diff:
            assert no == k, f"{what}: row {r}: short row must select every valid entry"
            sk = float(ora_scores[r, os_[k - 1]])
            tol = ATOL + RTOL * abs(sk)
            for j in diff:
                assert abs(float(ora_scores[r, j]) - sk) <= tol, \
                    f"{what}: row {r}: entry {j} (oracle {ora_scores[r, j]}) differs from the k-th score {sk}"
