#!/usr/bin/env python3
"""Benchmark of the CSA indexer hot path on one MI355X.

A step is one fused score + top-k selection (csa_index_select) over the
seq-16384 prefill workload: B=1, S=16384, H=64 heads, D=128, compress rate 4
(W=4096 compressed entries), top_k=512, Gaussian bf16 inputs, causal mask.
Inputs are resident in HBM before timing starts; the selection output is
int32 [S, 512] and the score matrix never reaches HBM.

value = causal score entries per second = (unmasked (i, j) pairs) / step time.
Also reported on the same line (each leg: HIP events around every call on
the launch stream, mean / median / min over the timed calls):
  roofline      the fused kernel's algorithmic flops (pairs * 2*H*D) per launch
                over its mean event duration, against the dense bf16 MFMA peak,
                and against the achievable MFMA rate measured in this run
  achievable    calibration kernels on the same GPU: a back-to-back bf16 MFMA
                loop on Gaussian and on zero operands (the chip lowers its clock
                under the higher switching power of Gaussian data), a streaming
                read and a copy of 1 GiB
  scores_only   csa_index_score on the same workload (fp32 [S,W] output)
  packed        the packed-document prefill (B=4, S=8192, W=2048, 1-6 documents
                per row, segment + causal mask), fused select
  decode        B=64 one-row decode over a 32768-entry cache (valid length
                U[4096,32768]): rows/s and HBM fraction of the algorithmic bytes
  backward      csa_index_score_backward on the prefill workload (dq, dk, dw for a
                Gaussian upstream gradient): algorithmic flops pairs * 6*H*D
  kl            csa_index_kl_loss on the prefill workload (fused, no gradient):
                the indexer's KL loss against a random target distribution
  cpu_baseline  the CPU oracle (scores + top-k) on a bounded sample of the
                prefill rows, and of the decode rows

Every leg first runs its step untimed for --settle-s seconds (default 0.5)
so that the GPU's clocks have ramped up under the load before the W warmup
and K timed steps; without it the first few dozen calls of a leg run up to
25 % slower and a short run times the ramp.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--settle-s S] [--legs ...]
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer score entries/sec (causal) + % bf16 MFMA peak; decode rows/sec + % HBM BW"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
CSRC = os.path.join(ROOT, "sparse_attention_indexer_csa_amd", "csrc")
CALIB_LIB = os.path.join(ROOT, "sparse_attention_indexer_csa_amd", "libcsa_calib.so")

# HBM bytes per call, from FETCH_SIZE and WRITE_SIZE counter runs scaled by
# what the same counters read for the calibration copy of 1 GiB (FETCH_SIZE
# x 1.99996, WRITE_SIZE x 1.0), summed over the kernels of the call.  Each
# entry is valid only for the kernel sources it was taken on (sha256 over the
# files its kernels are compiled from); reported as null otherwise.
FORWARD_SOURCES = ["csa_device.hpp", "csa_kernels.hip", "csa_launch.hpp", "csa_score.hpp", "csa_topk.hpp"]
BACKWARD_SOURCES = ["csa_backward.hip", "csa_backward.hpp", "csa_device.hpp", "csa_score.hpp"]
MEASURED_TRAFFIC = {
    "select": {"sources": FORWARD_SOURCES,
               "sha": "d2d37f996557ed10960dce85db9b54223ada86546d92d7ac68eab3c92e6de076",
               "kernels": ["rows3_kernel<128, 2, 2>"], "fetch_bytes": 289429128, "write_bytes": 33554432},
    "decode": {"sources": FORWARD_SOURCES,
               "sha": "d2d37f996557ed10960dce85db9b54223ada86546d92d7ac68eab3c92e6de076",
               "kernels": ["stream_kernel<128, 2>", "topk_block_kernel"], "fetch_bytes": 326239355,
               "write_bytes": 5109952},
    "backward": {"sources": BACKWARD_SOURCES,
                 "sha": "a7ca52bcf26cfb3fd8efe55801257ab8ae3597f7878ce3a36c165df0bb12e886",
                 "kernels": ["bwd_rows_kernel<128, 2>", "bwd_keys_kernel<128, 2>", "bwd_reduce_kernel"],
                 "fetch_bytes": 1499413736, "write_bytes": 882802688},
}

DEFAULT_LEGS = "calib,select,score,packed,decode,backward,kl,cpu"


def sources_sha(names=FORWARD_SOURCES):
    h = hashlib.sha256()
    for name in sorted(names):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(leg):
    """HBM bytes per call of the leg's kernels (fetch + write), or None when
    the counters were taken on other kernel sources."""
    t = MEASURED_TRAFFIC.get(leg)
    if t is None or t["sha"] != sources_sha(t["sources"]):
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def row_kernel_name(P):
    hb = 1 if P.H <= 32 else 2 if P.H <= 64 else 4
    return f"csa::rows3_kernel<{P.D}, {hb}, 2>" if hb <= 2 else f"csa::rows_kernel<{P.D}, {hb}, 2>"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--legs", default=DEFAULT_LEGS,
                    help="comma list of: calib, select, score, packed, decode, backward, kl, cpu")
    ap.add_argument("--settle-s", type=float, default=0.5,
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


def visible_pairs(P, rows=None, segments=True):
    """Unmasked (row, entry) pairs: entries before the causal threshold (and in
    the row's segment when segments are given and counted)."""
    rows = np.arange(P.B * P.S) if rows is None else np.asarray(rows)
    b, i = rows // P.S, rows % P.S
    off = P.q_offset[b].astype(np.int64) if P.q_offset is not None else 0
    thr = np.clip((off + i + 1) // P.m, 0, P.W)
    if P.q_seg is None or not segments:
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
    calls, then steps timed calls, each between two HIP events on the current
    stream (the stream the binding launches on).  Returns wall ms per step and
    the mean, median and min event ms per call."""
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
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    return dict(wall_ms=wall, ev_mean=float(ms.mean()), ev_median=float(np.median(ms)), ev_min=float(ms.min()))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def calibrate(torch, dev, steps, warmup):
    """Achievable rates on this GPU from the calibration kernels."""
    lib = ctypes.CDLL(CALIB_LIB)
    lib.csa_calib_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p]
    lib.csa_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                                   ctypes.c_void_p]
    lib.csa_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                   ctypes.c_void_p]
    for f in (lib.csa_calib_mfma_bf16, lib.csa_calib_read, lib.csa_calib_copy):
        f.restype = ctypes.c_int32
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = lambda: ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    out = {}
    # operands: Gaussian values scaled like the indexer's q and k, as bf16
    rng = np.random.default_rng(0)
    g = (rng.standard_normal(256 * 8).astype(np.float32) / np.float32(np.sqrt(128.0)))
    bits = ((g.view(np.uint32) + np.uint32(0x7FFF) + ((g.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
    ops = {"gauss": torch.from_numpy(bits.view(np.int16)).to(dev),
           "zeros": torch.zeros(256 * 8, dtype=torch.int16, device=dev)}
    blocks, iters = 8 * cus, 2000
    sink = torch.empty(blocks * 4, dtype=torch.float32, device=dev)
    flops = blocks * 4 * iters * 8 * 32768
    for name, o in ops.items():
        def step(_, o=o):
            st = lib.csa_calib_mfma_bf16(ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(sink.data_ptr()), blocks,
                                         iters, stream())
            if st != 0:
                raise RuntimeError(f"calibration MFMA launch failed ({st})")
        t = time_calls(step, max(3, steps // 4), warmup, torch)
        out[f"mfma_bf16_tflops_{name}"] = flops / (t["ev_median"] * 1e-3) / 1e12
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    rsink = torch.empty(8 * cus * 256, dtype=torch.int32, device=dev)

    def step_r(_):
        if lib.csa_calib_read(ctypes.c_void_p(src.data_ptr()), n, ctypes.c_void_p(rsink.data_ptr()), 8 * cus,
                              stream()) != 0:
            raise RuntimeError("calibration read launch failed")

    def step_c(_):
        if lib.csa_calib_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n, 8 * cus,
                              stream()) != 0:
            raise RuntimeError("calibration copy launch failed")

    t = time_calls(step_r, max(3, steps // 4), warmup, torch)
    out["hbm_read_GBs"] = n / (t["ev_median"] * 1e-3) / 1e9
    t = time_calls(step_c, max(3, steps // 4), warmup, torch)
    out["hbm_copy_GBs"] = 2 * n / (t["ev_median"] * 1e-3) / 1e9
    out["copy_bytes_read"] = n
    out["copy_bytes_written"] = n
    out["note"] = ("MFMA loop: 8 workgroups of 4 waves per CU, back-to-back v_mfma_f32_32x32x16_bf16 on 4 "
                   "accumulators; read/copy: 1 GiB, 16-byte accesses, 8 workgroups per CU; median event time")
    del src, dst
    return out


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

    achievable = None
    if "calib" in legs:
        log("calibration legs (MFMA loop, read, copy)")
        achievable = calibrate(torch, dev, args.steps, args.warmup)
        result["achievable"] = achievable

    if "select" in legs:
        def step(_):
            csa.select(d["q"], d["k"], d["w"], P.top_k, P.m, out=out_idx)

        log(f"select: {args.warmup} warmup + {args.steps} timed steps")
        t = time_calls(step, args.steps, args.warmup, torch)
        result["value"] = pairs / (t["wall_ms"] * 1e-3)
        result["ms_per_step"] = t["wall_ms"]
        achieved = flops / (t["ev_mean"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic("select"),
                "kernel": row_kernel_name(P), "kernel_ms_mean": t["ev_mean"], "kernel_ms_median": t["ev_median"],
                "kernel_ms_min": t["ev_min"], "flops_per_launch": flops, "sources_sha": sources_sha()[:16]}
        if achievable:
            ach = achievable["mfma_bf16_tflops_gauss"]
            roof["achievable_peak"] = ach
            roof["frac_of_achievable"] = achieved / ach
        result["roofline"] = roof
        log(f"select: {t['wall_ms']:.3f} ms/step, kernel mean {t['ev_mean']:.3f} median {t['ev_median']:.3f} "
            f"min {t['ev_min']:.3f} ms, {achieved:.1f} TFLOP/s")

    if "score" in legs:
        out_s = torch.empty((P.B, P.S, P.W), dtype=torch.float32, device=dev)

        def step_s(_):
            csa.score(d["q"], d["k"], d["w"], P.m, out=out_s)

        log("scores-only leg")
        t = time_calls(step_s, args.steps, args.warmup, torch)
        ach = flops / (t["ev_mean"] * 1e-3) / 1e12
        result["scores_only"] = {"entries_per_s": pairs / (t["wall_ms"] * 1e-3), "ms_per_step": t["wall_ms"],
                                 "kernel_ms_mean": t["ev_mean"], "kernel_ms_median": t["ev_median"],
                                 "kernel_ms_min": t["ev_min"], "tflops": ach, "mfma_frac": ach / PEAK_BF16_TFLOPS,
                                 "output": "fp32 [S,W] = %d MiB" % (P.S * P.W * 4 >> 20)}
        del out_s

    if "kl" in legs:
        gen = torch.Generator(device=dev).manual_seed(17)
        target = torch.rand((P.B, P.S, P.W), generator=gen, device=dev, dtype=torch.float32)
        kl_out = torch.empty((P.B, P.S), dtype=torch.float32, device=dev)

        def step_kl(_):
            csa.kl_loss(d["q"], d["k"], d["w"], target, P.m, out=kl_out)

        log("kl leg")
        t = time_calls(step_kl, args.steps, args.warmup, torch)
        ach = flops / (t["ev_mean"] * 1e-3) / 1e12
        result["kl"] = {"workload": "indexer KL loss, fused (no gradient), random target, " + CONFIG_TITLES["c3"],
                        "entries_per_s": pairs / (t["wall_ms"] * 1e-3), "ms_per_step": t["wall_ms"],
                        "kernel_ms_mean": t["ev_mean"], "kernel_ms_median": t["ev_median"],
                        "kernel_ms_min": t["ev_min"], "tflops": ach, "mfma_frac": ach / PEAK_BF16_TFLOPS}
        del target, kl_out

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
        t = time_calls(step_b, args.steps, args.warmup, torch)
        bflops = pairs * 6 * P.H * P.D
        ach = bflops / (t["ev_mean"] * 1e-3) / 1e12
        result["backward"] = {"workload": "gradients dq, dk, dw of sum(g * score) on " + CONFIG_TITLES["c3"],
                              "entries_per_s": pairs / (t["wall_ms"] * 1e-3), "ms_per_step": t["wall_ms"],
                              "call_ms_mean": t["ev_mean"], "call_ms_median": t["ev_median"],
                              "call_ms_min": t["ev_min"], "flops_per_call": bflops, "tflops": ach,
                              "mfma_frac": ach / PEAK_BF16_TFLOPS, "workspace_bytes": wsb.numel(),
                              "traffic": measured_traffic("backward")}
        log(f"backward: {t['wall_ms']:.3f} ms/step, call {t['ev_mean']:.3f} ms, {ach:.1f} TFLOP/s")
        del g, dq, dk, dw, wsb

    del d
    if "packed" in legs:
        Pp = make_config("c4")
        dp = to_device(Pp, dev)
        seg_pairs = visible_pairs(Pp)
        causal_pairs = visible_pairs(Pp, segments=False)
        out_p = torch.empty((Pp.B, Pp.S, Pp.top_k), dtype=torch.int32, device=dev)

        def step_p(_):
            csa.select(dp["q"], dp["k"], dp["w"], Pp.top_k, Pp.m, q_seg=dp["q_seg"], k_seg=dp["k_seg"], out=out_p)

        log("packed-document leg")
        t = time_calls(step_p, args.steps, args.warmup, torch)
        ach = seg_pairs * 2 * Pp.H * Pp.D / (t["ev_mean"] * 1e-3) / 1e12
        result["packed"] = {"workload": CONFIG_TITLES["c4"] + ", fused select, seed 4",
                            "entries_per_s": seg_pairs / (t["wall_ms"] * 1e-3), "ms_per_step": t["wall_ms"],
                            "kernel_ms_mean": t["ev_mean"], "kernel_ms_median": t["ev_median"],
                            "kernel_ms_min": t["ev_min"], "same_segment_pairs": seg_pairs,
                            "causal_pairs": causal_pairs, "tflops": ach, "mfma_frac": ach / PEAK_BF16_TFLOPS}
        del dp, out_p, Pp

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
        t = time_calls(step_d, args.steps, args.warmup, torch)
        gbs = alg_bytes / (t["ev_mean"] * 1e-3) / 1e9
        dec = {"workload": CONFIG_TITLES["c5"], "rows_per_s": Pd.B / (t["wall_ms"] * 1e-3),
               "ms_per_step": t["wall_ms"], "call_ms_mean": t["ev_mean"], "call_ms_median": t["ev_median"],
               "call_ms_min": t["ev_min"], "algorithmic_bytes": alg_bytes, "GB_s": gbs,
               "hbm_frac": gbs / PEAK_HBM_GBS, "plan": csa.resolve_plan(dd["q"], dd["k"], dd["w"], Pd.m),
               "traffic": measured_traffic("decode")}
        if achievable:
            dec["hbm_frac_of_achievable_read"] = gbs / achievable["hbm_read_GBs"]
        result["decode"] = dec
        del caches, dd, ws

    if "cpu" in legs:
        import oracle

        cpu = {"unit": "entries/s", "cores": oracle.threads(), "host_cpus_visible": len(os.sched_getaffinity(0)),
               "cpu_model": cpu_model(), "kind": "oracle"}
        rows = np.arange(0, P.S, args.cpu_row_stride)
        sample_pairs = visible_pairs(P, rows)
        log(f"cpu baseline: oracle on {len(rows)} rows ({sample_pairs} pairs), {oracle.threads()} threads")
        t0 = time.perf_counter()
        oracle.select(P, rows)
        dt = time.perf_counter() - t0
        cpu.update(value=sample_pairs / dt, seconds=dt,
                   sample=f"one query row in {args.cpu_row_stride} of the seq-16384 prefill "
                          f"({len(rows)} rows, {sample_pairs} causal pairs), scores + top-k")
        Pd = make_config("c5")
        drows = np.arange(0, Pd.B, 4)
        t0 = time.perf_counter()
        oracle.select(Pd, drows)
        dtd = time.perf_counter() - t0
        cpu["decode"] = {"rows_per_s": len(drows) / dtd, "seconds": dtd,
                         "sample": f"every 4th decode row ({len(drows)} of {Pd.B}), scores + top-k"}
        result["cpu_baseline"] = cpu

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
