"""Build libpgq.so (HIP, gfx950) in-tree with hipcc.

    python -m int6_weight_export_amd.build          # or build_library() from Python

Every translation unit is compiled to an object in parallel (the kernel instantiations are
spread over several units for that reason), then the objects are linked.  Objects go to
`_build/` next to this file; `incremental=True` reuses an object that is newer than its
source and every header.

Flags: strict IEEE binary32 (no FMA contraction, no fast-math, correctly rounded
divide/sqrt, fp32 denormals kept) because outputs are compared bit for bit; packed
fp32 instructions disabled.
"""
from __future__ import annotations

import glob
import json
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpgq.so")
OBJ_DIR = os.path.join(HERE, "_build")
SOURCES = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
HEADERS = sorted(glob.glob(os.path.join(HERE, "csrc", "*.h"))) + [os.path.join(ROOT, "include", "pgq.h")]
ARCH = os.environ.get("PGQ_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
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


def _jobs() -> int:
    env = os.environ.get("MAX_JOBS")
    n = int(env) if env and env.isdigit() else (os.cpu_count() or 4)
    return max(1, min(n, 16, len(SOURCES)))


RESOURCES = os.path.join(OBJ_DIR, "resources.json")
_FIELDS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch", "Occupancy [waves/SIMD]": "occupancy",
           "VGPRs Spill": "vgpr_spill", "SGPRs Spill": "sgpr_spill"}


def _resources(remarks: str) -> dict:
    """Per-kernel register, scratch and occupancy figures from the compiler's resource-usage
    remarks (-Rpass-analysis=kernel-resource-usage)."""
    out, name = {}, None
    for ln in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", ln)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z][^:]*): (\d+) \[-Rpass-analysis", ln)
        if m and name and m.group(1) in _FIELDS:
            out[name][_FIELDS[m.group(1)]] = int(m.group(2))
    return out


def _compile(src: str, incremental: bool, verbose: bool) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src)[:-4] + ".o")
    res = obj[:-2] + ".resources.json"
    if incremental and os.path.exists(obj) and os.path.exists(res):
        newest = max(os.path.getmtime(p) for p in [src, *HEADERS, __file__])
        if os.path.getmtime(obj) > newest:
            return obj
    cmd = [hipcc(), *HIPCC_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-I", os.path.join(ROOT, "include"), "-c",
           "-o", obj + ".tmp", src]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stderr)
        raise subprocess.CalledProcessError(r.returncode, cmd)
    with open(res, "w") as f:
        json.dump(_resources(r.stderr), f, indent=0)
    os.replace(obj + ".tmp", obj)
    return obj


def build_library(verbose: bool = False, incremental: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(_jobs()) as pool:
        objs = list(pool.map(lambda s: _compile(s, incremental, verbose), SOURCES))
    merged = {}
    for o in objs:
        with open(o[:-2] + ".resources.json") as f:
            merged.update(json.load(f))
    with open(RESOURCES, "w") as f:
        json.dump(merged, f, indent=0)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv, incremental="-i" in sys.argv))
