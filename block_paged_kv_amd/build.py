"""Build libpagedkv.so in-tree: HIP sources with hipcc for gfx950, host C++ with g++.

Usage: ``python block_paged_kv_amd/build.py`` (run the file, not the module:
importing the package loads the library this script builds).
Every call recompiles every source, so the library always matches the tree.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libpagedkv.so")

HIP_SOURCES = ["runtime.hip", "kv_copy.hip", "decode.hip", "prefill.hip", "mixed.hip"]
CXX_SOURCES = ["status.cpp", "allocator.cpp"]

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # Keep hipcc from forming packed-fp32 VALU ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
]
# Per-source additions. The prefill kernel takes finite inputs only: without
# NaN semantics its row maxima need no operand canonicalisation.
# decode.hip: matrix-core results in ordinary vector registers (the stage
# loop's accumulators would otherwise be copied between register files every
# stage).
HIP_EXTRA = {"prefill.hip": ["-fno-honor-nans"],
             "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # hipcc's host pass does not know the packed-fp32 feature name; that note is harmless.
    lines = [x for x in out.splitlines() if "packed-fp32-ops" not in x]
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n  " + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link ``libpagedkv.so``; return its path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    steps = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        steps.append([HIPCC, *HIP_FLAGS, *HIP_EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    cxx = shutil.which("g++") or "g++"
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        steps.append([cxx, *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        for msg in ex.map(_run, steps):
            if verbose and msg:
                print(msg)
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
