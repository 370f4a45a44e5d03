"""Builds libspkv.so for gfx950 in-tree.

    python shared_prefix_paged_amd/build.py   (runs without importing the package)

Host sources are compiled with g++ (no HIP dependency); the HIP sources with
hipcc for gfx950 only, with packed-fp32 code generation disabled; everything
is linked by hipcc into ``shared_prefix_paged_amd/libspkv.so``.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libspkv.so")

HOST_SOURCES = ["alloc.cpp", "plan.cpp"]
HIP_SOURCES = ["kernels.hip", "probes.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libspkv.so)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run(["g++", "-std=c++17", "-O2", "-fPIC", "-Wall", "-Wextra", f"-I{INCLUDE}", "-c",
              os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run([hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              # MFMA accumulators in ordinary VGPRs: the softmax rescales them in place
              "-mllvm", "-amdgpu-mfma-vgpr-form=1",
              "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
