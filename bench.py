#!/usr/bin/env python3
"""Benchmark of the CSA indexer hot path on one MI355X.

A step is one fused score + top-k selection (csa_index_select) over the
seq-16384 prefill workload: B=1, S=16384, H=64 heads, D=128, compress rate 4
(W=4096 compressed entries), top_k=512, Gaussian bf16 inputs, causal mask.
Inputs are resident in HBM before timing starts; the selection output is
int32 [S, 512] and the score matrix never reaches HBM.

value = causal score entries per second = (unmasked (i, j) pairs) / step time.
Also reported on the same line:
  roofline      the fused kernel's algorithmic flops (pairs * 2*H*D) per launch
                over its mean HIP-event duration, against the dense bf16 MFMA peak
  scores_only   csa_index_score on the same workload (fp32 [S,W] output)
  decode        B=64 one-row decode over a 32768-entry cache (valid length
                U[4096,32768]): rows/s and HBM fraction of the algorithmic bytes
  backward      csa_index_score_backward on the same workload (dq, dk, dw for a
                Gaussian upstream gradient): algorithmic flops pairs * 6*H*D
                (logit recompute, dq and dk products) over the call's duration
  cpu_baseline  the CPU oracle (scores + top-k) on a bounded sample of the rows
  copy          (leg "copy", off by default) a plain 1 GiB device copy, the
                calibration kernel for the FETCH_SIZE / WRITE_SIZE counters

Every leg first runs its step untimed for --settle-s seconds (default 0.5)
so that the GPU's clocks have ramped up under the load before the W warmup
and K timed steps; without it the first few dozen calls of a leg run up to
25 % slower and a short run times the ramp.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--settle-s S]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer score entries/sec (causal) + % bf16 MFMA peak; decode rows/sec + % HBM BW"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
CSRC = os.path.join(ROOT, "sparse_attention_indexer_csa_amd", "csrc")

# HBM bytes per launch of the fused prefill kernel, from FETCH_SIZE and
# WRITE_SIZE counter runs scaled by what the same counters read for a plain
# copy of known size.  Valid only for the kernel sources they were taken on
# (sha256 over the files the forward kernels are compiled from); reported as
# null otherwise.
MEASURED_TRAFFIC = {
    "sources_sha": "fe00158dc0c145c04f73acd6e783eddb5b354a88a76bea612039acaa31286e6a",
    # FETCH_SIZE 139986.3 KiB x 1.99995 (copy calibration) + WRITE_SIZE 32768 KiB x 1.0
    "bytes_per_launch": 320_239_000,
}


FORWARD_SOURCES = ["csa_device.hpp", "csa_kernels.hip", "csa_launch.hpp", "csa_score.hpp", "csa_topk.hpp"]


def sources_sha():
    h = hashlib.sha256()
    for name in sorted(FORWARD_SOURCES):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic():
    t = MEASURED_TRAFFIC
    if t is None or t["sources_sha"] != sources_sha():
        return None
    return t["bytes_per_launch"]


def row_kernel_name(P):
    hb = 1 if P.H <= 32 else 2 if P.H <= 64 else 4
    return f"csa::rows_kernel<{P.D}, {hb}, 2>"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--legs", default="select,score,decode,backward,cpu",
                    help="comma list of: select, score, decode, backward, cpu, copy")
    ap.add_argument("--settle-s", type=float, default=SETTLE_S,
                    help="untimed seconds of calls before each leg's warmup (clock ramp); 0 disables")
    ap.add_argument("--cpu-row-stride", type=int, default=2,
                    help="the CPU baseline runs every n-th row of the prefill workload")
    return ap.parse_args()


def to_device(P, dev):
    import torch

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def i32(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)

    return dict(q=bf16(P.q), k=bf16(P.k), w=bf16(P.w), q_offset=i32(P.q_offset), q_seg=i32(P.q_seg),
                k_seg=i32(P.k_seg))


def visible_pairs(P, rows=None):
    """Unmasked (row, entry) pairs: entries before the causal threshold (and in
    the row's segment when segments are given)."""
    rows = np.arange(P.B * P.S) if rows is None else np.asarray(rows)
    b, i = rows // P.S, rows % P.S
    off = P.q_offset[b].astype(np.int64) if P.q_offset is not None else 0
    thr = np.clip((off + i + 1) // P.m, 0, P.W)
    if P.q_seg is None:
        return int(thr.sum())
    total = 0
    for bb in np.unique(b):
        sel = b == bb
        ks = P.k_seg[bb]
        ids = np.unique(ks)
        cum = {s: np.concatenate([[0], np.cumsum(ks == s)]) for s in ids}
        for ii, tt in zip(i[sel], thr[sel]):
            s = P.q_seg[bb, ii]
            total += int(cum[s][tt]) if s in cum else 0
    return total


SETTLE_S = 0.5


def time_calls(fn, steps, warmup, torch):
    """Runs fn untimed for SETTLE_S seconds of wall time (the GPU raises its
    clocks over the first tens of milliseconds under load, so a short warmup
    would time the ramp instead of the steady state), then warmup more untimed
    calls, then steps timed calls; returns (wall ms per step, mean event ms
    per call)."""
    t_end = time.perf_counter() + SETTLE_S
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn(0)
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        evs[s][0].record()
        fn(s)
        evs[s][1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ev = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    return wall, ev


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the indexer would shard by batch or by rows with no communication between GPUs)", file=sys.stderr)
        sys.exit(2)
    legs = set(args.legs.split(","))
    global SETTLE_S
    SETTLE_S = max(0.0, args.settle_s)

    import torch

    import sparse_attention_indexer_csa_amd as csa
    from synth import CONFIG_TITLES, make_config

    csa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    P = make_config("c3")
    d = to_device(P, dev)
    pairs = visible_pairs(P)
    flops = pairs * 2 * P.H * P.D
    out_idx = torch.empty((P.B, P.S, P.top_k), dtype=torch.int32, device=dev)
    result = {
        "metric": METRIC, "value": None, "unit": "entries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "seq-16384 prefill, fused score + top-k select: " + CONFIG_TITLES["c3"],
                   "B": P.B, "S": P.S, "H": P.H, "D": P.D, "W": P.W, "compress_rate": P.m, "top_k": P.top_k,
                   "mask": "causal", "inputs": "Gaussian bf16, seed 3", "causal_pairs": pairs,
                   "plan": csa.resolve_plan(d["q"], d["k"], d["w"], P.m)},
    }

    if "select" in legs:
        def step(_):
            csa.select(d["q"], d["k"], d["w"], P.top_k, P.m, out=out_idx)

        log(f"select: {args.warmup} warmup + {args.steps} timed steps")
        wall, ev = time_calls(step, args.steps, args.warmup, torch)
        result["value"] = pairs / (wall * 1e-3)
        result["ms_per_step"] = wall
        achieved = flops / (ev * 1e-3) / 1e12
        result["roofline"] = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                              "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(),
                              "kernel": row_kernel_name(P), "kernel_ms": ev,
                              "flops_per_launch": flops, "sources_sha": sources_sha()[:16]}
        log(f"select: {wall:.3f} ms/step, kernel {ev:.3f} ms, {achieved:.1f} TFLOP/s")

    if "score" in legs:
        out_s = torch.empty((P.B, P.S, P.W), dtype=torch.float32, device=dev)

        def step_s(_):
            csa.score(d["q"], d["k"], d["w"], P.m, out=out_s)

        log("scores-only leg")
        wall, ev = time_calls(step_s, args.steps, args.warmup, torch)
        ach = flops / (ev * 1e-3) / 1e12
        result["scores_only"] = {"entries_per_s": pairs / (wall * 1e-3), "ms_per_step": wall, "kernel_ms": ev,
                                 "tflops": ach, "mfma_frac": ach / PEAK_BF16_TFLOPS,
                                 "output": "fp32 [S,W] = %d MiB" % (P.S * P.W * 4 >> 20)}
        del out_s

    if "decode" in legs:
        Pd = make_config("c5")
        dd = to_device(Pd, dev)
        # a second cache at another address so the 256 MB last-level cache
        # cannot serve the next step's keys
        caches = [dd["k"], dd["k"].clone()]
        L = Pd.meta["valid_len"]
        alg_bytes = int(L.sum()) * Pd.D * 2 + Pd.B * Pd.H * Pd.D * 2 + Pd.B * Pd.H * 2 + Pd.B * Pd.top_k * 4 + Pd.B * 4
        ws = torch.empty(csa.workspace_size(dd["q"], dd["k"], dd["w"], Pd.top_k, Pd.m), dtype=torch.uint8,
                         device=dev)
        out_d = torch.empty((Pd.B, 1, Pd.top_k), dtype=torch.int32, device=dev)

        def step_d(s):
            csa.select(dd["q"], caches[s % 2], dd["w"], Pd.top_k, Pd.m, q_offset=dd["q_offset"], out=out_d,
                       workspace=ws)

        log("decode leg")
        wall, ev = time_calls(step_d, args.steps, args.warmup, torch)
        gbs = alg_bytes / (ev * 1e-3) / 1e9
        result["decode"] = {"workload": CONFIG_TITLES["c5"], "rows_per_s": Pd.B / (wall * 1e-3),
                            "ms_per_step": wall, "call_ms": ev, "algorithmic_bytes": alg_bytes, "GB_s": gbs,
                            "hbm_frac": gbs / PEAK_HBM_GBS,
                            "plan": csa.resolve_plan(dd["q"], dd["k"], dd["w"], Pd.m)}
        del caches, dd, ws

    if "backward" in legs:
        # gradient of sum(g * score) for a Gaussian upstream gradient g [B,S,W]
        gen = torch.Generator(device=dev).manual_seed(13)
        g = torch.randn((P.B, P.S, P.W), generator=gen, device=dev, dtype=torch.float32)
        dq = torch.empty((P.B, P.H, P.S, P.D), dtype=torch.float32, device=dev)
        dk = torch.empty((P.B, P.W, P.D), dtype=torch.float32, device=dev)
        dw = torch.empty((P.B, P.S, P.H), dtype=torch.float32, device=dev)
        wsb = torch.empty(csa.backward_workspace_size(d["q"], d["k"], d["w"], P.m), dtype=torch.uint8, device=dev)

        def step_b(_):
            csa.score_backward(d["q"], d["k"], d["w"], g, P.m, workspace=wsb, dq=dq, dk=dk, dw=dw)

        log("backward leg")
        wall, ev = time_calls(step_b, args.steps, args.warmup, torch)
        bflops = pairs * 6 * P.H * P.D
        ach = bflops / (ev * 1e-3) / 1e12
        result["backward"] = {"workload": "gradients dq, dk, dw of sum(g * score) on " + CONFIG_TITLES["c3"],
                              "entries_per_s": pairs / (wall * 1e-3), "ms_per_step": wall, "call_ms": ev,
                              "flops_per_call": bflops, "tflops": ach, "mfma_frac": ach / PEAK_BF16_TFLOPS,
                              "workspace_bytes": wsb.numel()}
        log(f"backward: {wall:.3f} ms/step, call {ev:.3f} ms, {ach:.1f} TFLOP/s")
        del g, dq, dk, dw, wsb

    if "copy" in legs:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)

        def step_c(_):
            dst.copy_(src)

        log("copy leg")
        wall, ev = time_calls(step_c, args.steps, args.warmup, torch)
        result["copy"] = {"bytes_read": n, "bytes_written": n, "call_ms": ev, "GB_s": 2 * n / (ev * 1e-3) / 1e9}
        del src, dst

    if "cpu" in legs:
        import oracle

        rows = np.arange(0, P.S, args.cpu_row_stride)
        sample_pairs = visible_pairs(P, rows)
        log(f"cpu baseline: oracle on {len(rows)} rows ({sample_pairs} pairs), {oracle.threads()} threads")
        t0 = time.perf_counter()
        oracle.select(P, rows)
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": sample_pairs / dt, "unit": "entries/s", "cores": oracle.threads(),
                                  "kind": "oracle", "seconds": dt,
                                  "sample": f"every {args.cpu_row_stride}th query row of the seq-16384 prefill "
                                            f"({len(rows)} rows, {sample_pairs} causal pairs), scores + top-k"}

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
