"""Builds libcsa_index.so (the HIP kernels + the C ABI) and libcsa_calib.so
(the benchmark's calibration kernels) in place, for gfx950.

    python -m sparse_attention_indexer_csa_amd.build

hipcc cross-compiles without a GPU.  Packed fp32 vector instructions are
switched off for all device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libcsa_index.so")

SOURCES = ["csa_kernels.hip", "csa_backward.hip", "csa_api.cpp"]
# Calibration kernels for the benchmark's achievable peaks (include/csa_calib.h).
CALIB_DIR = os.path.join(HERE, "calib")
CALIB_SOURCE = "csa_calib.hip"
CALIB_LIB = os.path.join(HERE, "libcsa_calib.so")
HEADERS = ["csa_device.hpp", "csa_score.hpp", "csa_topk.hpp", "csa_launch.hpp", "csa_backward.hpp"]

ARCH = os.environ.get("CSA_INDEX_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set ROCM_PATH)")


FLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: no AGPR <-> VGPR copies before the epilogue
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
NOISE = "'-packed-fp32-ops' is not a recognized feature"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libcsa_index.so")
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if ln.strip() and NOISE not in ln]
    if msgs and verbose:
        print("\n".join(msgs))


def build(verbose: bool = False) -> str:
    """Compile the library and the calibration library (always, every source
    in parallel) and return the library's path."""
    tag = f".tmp{os.getpid()}"
    objs = [os.path.join(CSRC, s + tag + ".o") for s in SOURCES]
    calib_obj = os.path.join(CALIB_DIR, CALIB_SOURCE + tag + ".o")
    jobs = [(os.path.join(CSRC, s), o) for s, o in zip(SOURCES, objs)]
    jobs.append((os.path.join(CALIB_DIR, CALIB_SOURCE), calib_obj))
    outs = [(LIB, objs), (CALIB_LIB, [calib_obj])]
    try:
        with ThreadPoolExecutor(len(jobs)) as ex:
            list(ex.map(lambda so: _run([hipcc(), *FLAGS, "-c", so[0], "-o", so[1]], verbose), jobs))
        for lib, lib_objs in outs:
            _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *lib_objs, "-o", lib + tag], verbose)
            os.replace(lib + tag, lib)
    finally:
        for o in objs + [calib_obj] + [lib + tag for lib, _ in outs]:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
