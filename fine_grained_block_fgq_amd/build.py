"""Build libfgq.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfgq.so")
SOURCES = ["quant.hip", "gemm.hip", "nvfp4.hip", "api.cpp"]
# the measurement library (ceiling kernels and the FP8-MFMA accuracy probe): not the method
CALIB_LIB = os.path.join(HERE, "libfgq_calib.so")
CALIB_SOURCES = ["calib.hip", "calib_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32: keep denormals, no contraction of separate multiplies and adds
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
    "-Wno-inline-asm",
]


def _build_one(sources, lib, verbose):
    srcs = []
    for s in sources:
        path = os.path.join(CSRC, s)
        # hipcc compiles .cpp as host code; mark every source as HIP
        srcs += ["-x", "hip", path] if s.endswith(".cpp") else [path]
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Build libfgq.so (the method) and libfgq_calib.so (measurement only); returns the
    former's path."""
    _build_one(SOURCES, LIB, verbose)
    _build_one(CALIB_SOURCES, CALIB_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
