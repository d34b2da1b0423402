"""Build libglq.so in-tree: hipcc for the gfx950 kernels, g++ for host code.

Usage: python -m dequant_e8_codebook_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INC = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "lib")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(OUT_DIR, "libglq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HOST_SOURCES = ["glq_codebook.cpp", "glq_encode.cpp", "glq_ep.cpp"]
HIP_SOURCES = ["glq_kernels.hip"]


def _run(cmd):
    print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = True) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    common = ["-std=c++17", "-fPIC", "-I" + INC, "-I" + CSRC]
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run(["g++", "-O2", "-Wall", "-pthread"] + common + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run([HIPCC, "-O3", "--offload-arch=" + ARCH,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
             + common + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-pthread", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
