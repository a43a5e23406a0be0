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


HIP_SOURCES = ["kern_q8g64.hip", "kern_q4g32.hip", "kern_q8g128.hip", "kern_q8pc.hip",
               "kern_q4g32_swiglu.hip", "kern_argmax_epi.hip", "kern_mma.hip", "argmax.hip", "read_stream.hip",
               "launch.hip",
               "abi.cpp"]
HOST_SOURCES = ["qpack.cpp"]


def build(verbose: bool = True) -> str:
    """Compiles every source (the per-format kernel units in parallel) and
    links libqgemv.so."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        jobs.append((obj, [HIPCC] + HIP_FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]))
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        jobs.append((obj, ["g++"] + HOST_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]))
    workers = max(1, min(len(jobs), len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda job: _run(job[1]), jobs))
    objs = [obj for obj, _ in jobs]
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
