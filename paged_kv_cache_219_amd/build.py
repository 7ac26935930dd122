"""Build libpa.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_219_amd.build [--jobs N]

Every source is compiled on every call (no staleness logic), objects go to
``_build/`` at the repository root, the shared library to
``paged_kv_cache_219_amd/libpa.so``.  Device code is compiled with packed-fp32
instructions disabled.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["allocator.cpp", "prefix_plan.cpp", "cache_ops.hip", "decode.hip", "prefill.hip",
           "mixed.hip"]

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include")]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


# Per-source extras.  The prefill and decode bodies never let a NaN reach
# arithmetic that matters (masked scores are replaced by -inf with a select,
# tail values are zeroed bitwise), so the matrix-core sources are built
# assuming no NaN operands: fmax then needs no canonicalising instruction per
# operand.
EXTRA = {"prefill.hip": ["-fno-honor-nans"], "mixed.hip": ["-fno-honor-nans"]}


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", *COMMON, *DEVICE, *EXTRA.get(src, []), "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, len(SOURCES))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    a = ap.parse_args()
    try:
        build(a.jobs, verbose=True)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
