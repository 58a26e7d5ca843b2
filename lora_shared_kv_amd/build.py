"""Build the native libraries in-tree.

libskv.so       the product: C ABI (runtime.cpp) + HIP kernels for gfx950.
libskv_host.so  the same host runtime linked with the null device backend, for
                metadata tests on machines without a GPU.

Run as ``python -m lora_shared_kv_amd.build`` or call ``build()``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 ops are turned off for every HIP translation unit. MFMA
# accumulators are kept in VGPRs (the VGPR form of the MFMA instructions): the
# kernels rescale them with vector ops, which cannot read AGPRs.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-Wno-unused-result"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I" + INCLUDE, "-I" + CSRC]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("build step failed: " + " ".join(cmd))
    if out.strip():
        sys.stderr.write(out + "\n")


def build(verbose: bool = True) -> None:
    os.makedirs(OUT, exist_ok=True)
    cxx = shutil.which("g++") or "g++"
    rt_o = os.path.join(OUT, "runtime.o")
    null_o = os.path.join(OUT, "backend_null.o")
    k_o = os.path.join(OUT, "kernels.o")
    steps = [
        [cxx] + CXX_FLAGS + ["-c", os.path.join(CSRC, "runtime.cpp"), "-o", rt_o],
        [cxx] + CXX_FLAGS + ["-c", os.path.join(CSRC, "backend_null.cpp"), "-o", null_o],
        [cxx, "-shared", "-o", os.path.join(PKG, "libskv_host.so"), rt_o, null_o],
        [HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, "kernels.hip"), "-o", k_o],
        [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", os.path.join(PKG, "libskv.so"),
         rt_o, k_o],
    ]
    for cmd in steps:
        if verbose:
            print("[build]", " ".join(os.path.basename(c) if i == 0 else c for i, c in enumerate(cmd)),
                  flush=True)
        _run(cmd)


ASAN_LIB = os.path.join(OUT, "libskv_host_asan.so")


def build_asan(verbose: bool = True) -> str:
    """The CPU build of the host runtime (null device backend) under
    AddressSanitizer and UndefinedBehaviorSanitizer, for the sanitized runs of
    the host-library tests; g++ only, no HIP code. Returns the library path.
    Loading it needs the sanitizer runtimes preloaded (LD_PRELOAD)."""
    os.makedirs(OUT, exist_ok=True)
    cxx = shutil.which("g++") or "g++"
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-I" + INCLUDE, "-I" + CSRC]
    cmd = [cxx] + flags + ["-shared", "-o", ASAN_LIB, os.path.join(CSRC, "runtime.cpp"),
                           os.path.join(CSRC, "backend_null.cpp")]
    if verbose:
        print("[build] " + " ".join(os.path.basename(c) if i == 0 else c for i, c in enumerate(cmd)), flush=True)
    _run(cmd)
    return ASAN_LIB


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "asan":
        build_asan()
    else:
        build()
