"""Build ``libkvattn.so`` (the C-ABI library) in-tree for gfx950.

Host-only code (validation, planning) is compiled with g++; the kernels and the entry points
that call the HIP runtime with hipcc for gfx950. Every HIP compile disables packed-fp32
instruction selection. The library lands next to this file, where the binding loads it.

Usage: ``python -m kv_cache_decode_split_amd.build`` (or ``build()`` from Python).
"""

from __future__ import annotations

import concurrent.futures
import json
import os
import re
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

# The split kernel's families compile in separate files so that the build runs them in parallel.
HIP_SOURCES = ["kv_attn_split_vector128.hip", "kv_attn_split_vector64.hip",
               "kv_attn_split_mfma128.hip", "kv_attn_split_mfma64.hip", "kv_attn_split_rows.hip",
               "kv_attn_kernels.hip", "kv_attn_api.hip", "kv_evict.hip", "kv_probe.hip"]
CXX_SOURCES = ["kv_attn_plan.cpp"]
# hipcc's per-kernel resource report (registers, spills, scratch), checked after every compile.
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"


class ScratchError(RuntimeError):
    """A kernel of the library would spill registers to scratch memory."""


def parse_resource_usage(text: str) -> list:
    """The per-kernel records of hipcc's resource-usage remarks in ``text``: one dict per kernel
    with its mangled name and the reported values (as strings) keyed by the remark's label."""
    records = []
    for line in text.splitlines():
        if "remark:" not in line or RESOURCE_REMARKS not in line:
            continue
        body = line.split("remark:", 1)[1].rsplit("[", 1)[0].strip()
        if body.startswith("Function Name:"):
            records.append({"name": body.split(":", 1)[1].strip()})
        elif records and ":" in body:
            key, value = body.rsplit(":", 1)
            records[-1][key.strip()] = value.strip()
    return records


def scratch_offenders(records: list) -> list:
    """Kernels that use scratch memory or spill vector registers (to scratch or to AGPRs)."""
    bad = []
    for r in records:
        scratch = int(r.get("ScratchSize [bytes/lane]", "0"))
        vspill = int(r.get("VGPRs Spill", "0"))
        if scratch != 0 or vspill != 0:
            bad.append(f"{r['name']}: scratch {scratch} bytes/lane, {vspill} VGPRs spilled")
    return bad


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


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source and link the library. Always rebuilds. Returns the library path.

    Fails (ScratchError) if any kernel spills registers or uses scratch memory: every kernel of
    the library is meant to run from registers and LDS alone, and the resource report of each
    compile is checked.
    """
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    cxx = os.environ.get("CXX", "g++")
    if jobs <= 0:
        jobs = max(1, min(8, os.cpu_count() or 1))
    steps = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        steps.append([hipcc, *HIP_FLAGS, RESOURCE_REMARKS, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        steps.append([cxx, *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    records = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, steps):
            records.extend(parse_resource_usage(out))
            # (the remarks' source excerpts are lines of the form "  123 | code" and "      | ^")
            rest = "\n".join(l for l in out.splitlines()
                             if RESOURCE_REMARKS not in l and not re.match(r"^\s*\d*\s*\|", l)
                             and not l.startswith("In file included from"))
            if verbose and rest.strip():
                print(rest)
    bad = scratch_offenders(records)
    if bad:
        raise ScratchError("kernels that spill registers:\n  " + "\n  ".join(bad))
    with open(os.path.join(BUILD_DIR, "resource_usage.jsonl"), "w") as f:
        for r in records:
            f.write(json.dumps(r) + "\n")
    objs = [os.path.join(BUILD_DIR, s + ".o") for s in HIP_SOURCES + CXX_SOURCES]
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
