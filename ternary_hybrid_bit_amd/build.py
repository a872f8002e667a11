"""Ahead-of-time build of libwal.so for gfx950 (MI355X), in-tree.

    python ternary_hybrid_bit_amd/build.py

compiles the host packer with g++ and the HIP kernels with hipcc, and links
``ternary_hybrid_bit_amd/libwal.so``.  Packed-fp32 VALU forms are disabled on
the device pass; the host pass does not know that target feature and warns,
which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libwal.so")
ARCH = os.environ.get("WAL_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_SOURCES = ["wal_gpu.hip", "wal_base3.hip", "wal_gemm.hip", "wal_rotate.hip", "wal_int4.hip"]
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    host_o = os.path.join(BUILD, "wal_host.o")
    steps = [["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-c", os.path.join(CSRC, "wal_host.cpp"), "-o", host_o]]
    objs = [host_o]
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        steps.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    # the translation units are independent: compile them side by side
    # (a few GB of memory each at most)
    workers = max(1, min(len(steps), os.cpu_count() or 1, 6))
    with ThreadPoolExecutor(workers) as pool:
        for f in [pool.submit(_run, cmd, verbose) for cmd in steps]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
