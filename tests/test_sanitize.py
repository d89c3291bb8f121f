"""The oracle and the C ABI's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

* oracle: tests/sanitize/oracle_driver.c runs every oracle entry point on
  seeded small problems and edge cases (empty caches, rows that see nothing,
  segments, offsets, samples, top-k above the row length, -inf/NaN, KL rows
  without target mass), every buffer allocated at its exact size; leak
  checking on.
* C ABI: tests/sanitize/api_driver.cpp drives csa_api.cpp (built with the
  sanitizers on its host code) through every refusal path and a seeded sweep
  of problem descriptors with extreme sizes and strides through the host-only
  queries; the kernel launchers are stubs (tests/sanitize/launch_stubs.cpp),
  and no call reaches a launch.

Any sanitizer report fails the run (-fno-sanitize-recover).
"""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "sparse_attention_indexer_csa_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-ffp-contract=off", *SAN,
          os.path.join(ROOT, "oracle", "csa_oracle.c"), os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=1")
    res = _run([exe, "600"], env=env, timeout=600)
    assert "all checks hold" in res.stdout


def test_c_abi_host_code_under_asan_ubsan(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clangxx)):
        pytest.skip("hipcc / clang++ not found")
    # the sanitizers apply to the host side only (device code is compiled as usual)
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    hip = [hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san, *inc]
    objs = []
    for src in (os.path.join(CSRC, "csa_api.cpp"), os.path.join(HERE, "launch_stubs.cpp")):
        o = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([*hip, "-c", src, "-o", o])
        objs.append(o)
    drv = str(tmp_path / "api_driver.o")
    _run([clangxx, "-std=c++17", "-O1", "-g", *SAN, *inc, "-c", os.path.join(HERE, "api_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "api_driver")
    _run([clangxx, *SAN[:1], drv, *objs, f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe])
    # the HIP runtime's own allocations are not this code's leaks
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    res = _run([exe, "50000"], env=env, timeout=600)
    assert "all expectations hold" in res.stdout
