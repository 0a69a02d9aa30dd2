"""Build libflashopt.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libflashopt.so")
SOURCES = [os.path.join(CSRC, "flashopt_kernels.hip"), os.path.join(CSRC, "flashopt_api.cpp")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # one IEEE rounding per written operation, correctly rounded / and sqrt,
    # fp32 subnormals kept
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


CHECK_SRC = os.path.join(ROOT, "tests", "hip", "fastmath_check.hip")
CHECK_LIB = os.path.join(ROOT, "tests", "hip", "libfastmath_check.so")


def build_check(verbose: bool = False) -> str:
    """The GPU test library that verifies the short exact arithmetic sequences (test-only)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = CHECK_LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", CSRC, CHECK_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, CHECK_LIB)
    return CHECK_LIB


def build(extra_flags: list[str] | None = None, verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *(extra_flags or []), "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    build_check(verbose=True)
