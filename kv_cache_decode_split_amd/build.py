"""Build ``libkvattn.so`` (the C-ABI library) in-tree for gfx950.

Host-only code (validation, planning) is compiled with g++; the kernels and the entry points
that call the HIP runtime with hipcc for gfx950. Every HIP compile disables packed-fp32
instruction selection. The library lands next to this file, where the binding loads it.

Usage: ``python -m kv_cache_decode_split_amd.build`` (or ``build()`` from Python).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libkvattn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]

HIP_SOURCES = ["kv_attn_kernels.hip", "kv_attn_api.hip", "kv_evict.hip", "kv_probe.hip"]
CXX_SOURCES = ["kv_attn_plan.cpp"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; that warning is expected.
    lines = [l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l]
    if proc.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link the library. Always rebuilds. Returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    cxx = os.environ.get("CXX", "g++")
    steps = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        steps.append([hipcc, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        steps.append([cxx, *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, steps):
            if verbose and out.strip():
                print(out)
    objs = [os.path.join(BUILD_DIR, s + ".o") for s in HIP_SOURCES + CXX_SOURCES]
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
