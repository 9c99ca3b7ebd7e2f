"""Builds libw4a8.so in-tree with hipcc for gfx950.

Usage: python -m moe_token_int8_amd.build   (or __graft_entry__.build()).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libw4a8.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_SOURCES = ["w4a8_kernels.hip", "w4a16_kernels.hip", "w4a8_moe_kernels.hip", "w4a8_moe_tile_kernels.hip",
               "w4a8_decode_kernels.hip"]
HOST_SOURCES = ["w4a8_host.cpp"]     # plain C++ (no device code): built with the host compiler
CXX = os.environ.get("CXX", "g++")

# Packed-FP32 VALU forms are disabled for all device code; the float epilogues are written
# as scalar fma chains.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wno-unused-function",
          "-Wno-unused-variable", "-Wno-unused-but-set-variable"]


def build(verbose: bool = False) -> str:
    objs, procs = [], []
    os.makedirs(os.path.join(PKG, "_build"), exist_ok=True)
    # the translation units compile concurrently (one process each)
    for src in HIP_SOURCES + HOST_SOURCES:
        obj = os.path.join(PKG, "_build", src + ".o")
        if src in HIP_SOURCES:
            cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        else:
            cmd = [CXX, *COMMON, "-pthread", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), cmd))
        objs.append(obj)
    failed = [cmd for p, cmd in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    # the INT8 MFMA peak and HBM streaming-read microbenchmarks (standalone programs; not part of
    # the library)
    mbs = [subprocess.Popen([HIPCC, "-O3", "-std=c++17", *DEVICE_FLAGS, os.path.join(PKG, "microbench", name + ".hip"),
                             "-o", os.path.join(PKG, "_build", name)]) for name in ("mfma_peak", "hbm_read")]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "-pthread", *DEVICE_FLAGS, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for mb in mbs:
        if mb.wait() != 0:
            raise subprocess.CalledProcessError(mb.returncode, mb.args)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
