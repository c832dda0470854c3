"""C-ABI checks of the eviction-selection entry points that need no GPU.

Every kv_evict_select call here fails validation before the library makes any HIP call.
"""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kv_evict.h")

E = pytest.importorskip("kv_cache_decode_split_amd.kv_evict",
                        reason="libkvattn.so not built (run python -m kv_cache_decode_split_amd.build)")
K = pytest.importorskip("kv_cache_decode_split_amd.kv_attn")


def test_header_declarations_are_all_exported():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(kv_evict_\w+)\s*\(", text)))
    assert declared == sorted(E.EXPORTED_SYMBOLS)
    out = subprocess.run(["nm", "-D", "--defined-only", K.LIB_PATH], capture_output=True, text=True)
    assert set(re.findall(r"\bT (kv_evict_\w+)", out.stdout)) == set(declared)


def test_params_layout_matches_the_header():
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "kv_evict.h"', "int main(void){",
             'printf("size %zu\\n", sizeof(kv_evict_params));']
    for f, _ in E.kv_evict_params._fields_:
        lines.append(f'printf("{f} %zu\\n", offsetof(kv_evict_params, {f}));')
    lines.append("return 0;}")
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "probe.c"), os.path.join(d, "probe")
        open(src, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    for line in out.splitlines():
        what, value = line.split()
        if what == "size":
            assert ctypes.sizeof(E.kv_evict_params) == int(value)
        else:
            assert getattr(E.kv_evict_params, what).offset == int(value), what


def test_workspace_size_follows_the_budget():
    fixed = 930048
    for L, H, N in [(2, 3, 10), (32, 32, 4096), (32, 8, 131072), (3, 5, 777)]:
        n, pool = L * H * N, L * H * (N - 1)
        for M in (0, L * H, L * H + pool, 10**12):  # the budget alone decides
            assert E.kv_evict_workspace_size(E.make_evict_params(L, H, N, M)) == 0, M
        for M in (L * H + 1, L * H + pool // 2, L * H + pool - 1):
            ws = E.kv_evict_workspace_size(E.make_evict_params(L, H, N, M))
            assert fixed + 16 * n <= ws <= fixed + 32 * (n + 256 * 16384), (L, H, N, M, ws)
    assert E.kv_evict_workspace_size(E.make_evict_params(1, 1, 1, 5)) == 0  # N = 1: no pool


@pytest.mark.parametrize("kw,status", [
    (dict(num_layers=0), K.KV_ATTN_ERR_SHAPE),
    (dict(num_heads=-1), K.KV_ATTN_ERR_SHAPE),
    (dict(num_tokens=0), K.KV_ATTN_ERR_SHAPE),
    (dict(current=10), K.KV_ATTN_ERR_SHAPE),
    (dict(current=-1), K.KV_ATTN_ERR_SHAPE),
    (dict(row_stride=9), K.KV_ATTN_ERR_SHAPE),
    (dict(budget=-1), K.KV_ATTN_ERR_VALUE),
    (dict(num_layers=1 << 16, num_heads=1 << 10, num_tokens=1 << 5), K.KV_ATTN_ERR_UNSUPPORTED),
])
def test_invalid_params_are_rejected_before_any_launch(kw, status):
    args = dict(num_layers=2, num_heads=3, num_tokens=10, budget=20, current=None, row_stride=None)
    args.update(kw)
    p = E.make_evict_params(**args)
    assert E.kv_evict_workspace_size(p) == 0
    fake = ctypes.c_void_p(4096)
    st = E._lib.kv_evict_select(fake, fake, None, ctypes.byref(p), fake, 1 << 30, None)
    assert st == status


def test_missing_pointers_and_workspace_are_rejected():
    p = E.make_evict_params(2, 3, 10, 20)
    fake = ctypes.c_void_p(4096)
    assert E._lib.kv_evict_select(None, fake, None, ctypes.byref(p), fake, 1 << 30, None) == K.KV_ATTN_ERR_NULL
    assert E._lib.kv_evict_select(fake, None, None, ctypes.byref(p), fake, 1 << 30, None) == K.KV_ATTN_ERR_NULL
    assert E._lib.kv_evict_select(fake, fake, None, None, fake, 1 << 30, None) == K.KV_ATTN_ERR_NULL
    need = E.kv_evict_workspace_size(p)
    assert E._lib.kv_evict_select(fake, fake, None, ctypes.byref(p), None, 0, None) == K.KV_ATTN_ERR_WORKSPACE
    assert E._lib.kv_evict_select(fake, fake, None, ctypes.byref(p), fake, need - 1, None) == K.KV_ATTN_ERR_WORKSPACE
    # misaligned scores, workspace or per-row counts
    odd = ctypes.c_void_p(4098)
    assert E._lib.kv_evict_select(odd, fake, None, ctypes.byref(p), fake, need, None) == K.KV_ATTN_ERR_UNSUPPORTED
    assert E._lib.kv_evict_select(fake, fake, odd, ctypes.byref(p), fake, need, None) == K.KV_ATTN_ERR_UNSUPPORTED
    assert E._lib.kv_evict_select(fake, fake, None, ctypes.byref(p), ctypes.c_void_p(4104), need, None) \
        == K.KV_ATTN_ERR_UNSUPPORTED


def test_simulated_launch_failure_reports_a_hip_error(monkeypatch):
    monkeypatch.setenv("KV_ATTN_FAULT", "launch")
    p = E.make_evict_params(2, 3, 10, 20)
    fake = ctypes.c_void_p(4096)
    need = E.kv_evict_workspace_size(p)
    assert E._lib.kv_evict_select(fake, fake, None, ctypes.byref(p), fake, need, None) == K.KV_ATTN_ERR_HIP
