"""Builds libcsa_index.so (the HIP kernels + the C ABI) in place, for gfx950.

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
    """Compile the library (always, every source in parallel) and return its path."""
    tag = f".tmp{os.getpid()}"
    objs = [os.path.join(CSRC, s + tag + ".o") for s in SOURCES]
    tmp = LIB + tag
    try:
        with ThreadPoolExecutor(len(SOURCES)) as ex:
            list(ex.map(lambda so: _run([hipcc(), *FLAGS, "-c", os.path.join(CSRC, so[0]), "-o", so[1]], verbose),
                        zip(SOURCES, objs)))
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
