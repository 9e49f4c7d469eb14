"""Builds libdyra.so in-tree: host C++ (g++) + gfx950 HIP kernels (hipcc).

Usage: python -m input_adaptive_rank_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdyra.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")

HOST_SOURCES = ["host_linalg.cpp", "prepare.cpp"]
HIP_SOURCES = ["dyra_kernels.hip"]
HEADERS = ["host_linalg.h", "spec.h", "device_common.h", "gemm_engine.h"]

HOST_FLAGS = ["-O3", "-fPIC", "-std=c++17", "-mavx2", "-mfma", "-Wall", "-Wno-unused-function"]
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
             # no packed-fp32 VALU instructions in any kernel
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compiles every source (always) and links libdyra.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        out = _run(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out:
            print(out)
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        out = _run([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out:
            print(out)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp, "-lpthread"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
