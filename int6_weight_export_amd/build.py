"""Build libpgq.so (HIP, gfx950) in-tree with hipcc.

    python -m int6_weight_export_amd.build          # or build_library() from Python

Flags: strict IEEE binary32 (no FMA contraction, no fast-math, correctly rounded
divide/sqrt, fp32 denormals kept) because outputs are compared bit for bit; packed
fp32 instructions disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpgq.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("pgq_api.hip", "pgq_kernels.hip", "pgq_gemm.hip")]
HEADERS = [os.path.join(HERE, "csrc", "pgq_desc.h"), os.path.join(ROOT, "include", "pgq.h")]
ARCH = os.environ.get("PGQ_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libpgq")


def build_library(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
