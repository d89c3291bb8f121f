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

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libcsa_index.so")

SOURCES = ["csa_kernels.hip", "csa_api.cpp"]
HEADERS = ["csa_device.hpp", "csa_score.hpp", "csa_topk.hpp", "csa_launch.hpp"]

ARCH = os.environ.get("CSA_INDEX_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set ROCM_PATH)")


def command(out: str = LIB, extra: list | None = None) -> list:
    return [
        hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA accumulators in VGPRs: no AGPR <-> VGPR copies before the epilogue
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", f"-I{CSRC}",
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out, *(extra or []),
    ]


def build(verbose: bool = False) -> str:
    """Compile the library (always) and return its path."""
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libcsa_index.so")
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if ln.strip() and noise not in ln]
    if msgs and verbose:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
