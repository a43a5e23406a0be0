"""Builds libqgemv.so (HIP kernels for gfx950 + host C ABI) in-tree.

Run as ``python -m weight_only_block_amd.build``.  hipcc cross-compiles the
gfx950 code objects without a GPU.  Every HIP source is compiled with the
packed-fp32 feature switched off (see the hipcc flags below).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqgemv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall"]


def _run(cmd):
    print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    kern_o = os.path.join(BUILD, "kernels.o")
    _run([HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, "kernels.hip"), "-o", kern_o])
    objs.append(kern_o)
    abi_o = os.path.join(BUILD, "abi.o")
    _run([HIPCC] + HIP_FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, "abi.cpp"), "-o", abi_o])
    objs.append(abi_o)
    qpack_o = os.path.join(BUILD, "qpack.o")
    _run(["g++"] + HOST_FLAGS + ["-c", os.path.join(CSRC, "qpack.cpp"), "-o", qpack_o])
    objs.append(qpack_o)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
