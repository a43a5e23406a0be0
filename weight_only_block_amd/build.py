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


# Host-sanitizer build (CPU tests only): AddressSanitizer and
# UndefinedBehaviorSanitizer on the host code (the packer, the C ABI's
# validation, the launch sizing), linked against clang's shared ASan
# runtime; the gfx950 device code is built as usual.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libasan"]


def build(verbose: bool = True, out_dir: str = None, sanitize: bool = False) -> str:
    """Compiles every source (the per-format kernel units in parallel) and
    links libqgemv.so (into the package, or into out_dir).  sanitize=True
    makes the host-sanitizer build; every source then goes through hipcc so
    that one ASan runtime serves the whole library."""
    from concurrent.futures import ThreadPoolExecutor

    obj_dir = os.path.join(out_dir, "obj") if out_dir else BUILD
    lib_path = os.path.join(out_dir, "libqgemv.so") if out_dir else LIB
    os.makedirs(obj_dir, exist_ok=True)
    jobs = []
    hip_flags = HIP_FLAGS + (SANITIZE_HOST if sanitize else [])
    for src in HIP_SOURCES + (HOST_SOURCES if sanitize else []):
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        jobs.append((obj, [HIPCC] + hip_flags + lang + ["-c", os.path.join(CSRC, src), "-o", obj]))
    if not sanitize:
        for src in HOST_SOURCES:
            obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
            jobs.append((obj, ["g++"] + HOST_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]))
    run = _run if verbose else (lambda cmd: subprocess.check_call(cmd, stdout=subprocess.DEVNULL,
                                                                  stderr=subprocess.DEVNULL))
    workers = max(1, min(len(jobs), len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda job: run(job[1]), jobs))
    objs = [obj for obj, _ in jobs]
    tmp = lib_path + ".tmp%d" % os.getpid()
    run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + (SANITIZE_HOST if sanitize else [])
        + ["-o", tmp] + objs)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    build()
    sys.exit(0)
