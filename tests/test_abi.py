"""C-ABI checks that need no GPU: exports, struct layout, planning and host-side error paths.

Every call here fails validation (or is a pure host function) before the library makes any HIP
call, so nothing touches a device.
"""

import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kv_attn.h")

K = pytest.importorskip("kv_cache_decode_split_amd.kv_attn",
                        reason="libkvattn.so not built (run python -m kv_cache_decode_split_amd.build)")

from tests import plan_cases as C  # noqa: E402


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kv_attn_\w+)\s*\(", text)))


def test_header_declarations_are_all_exported():
    declared = _declared_functions()
    assert declared == sorted(K.EXPORTED_SYMBOLS)
    lib = ctypes.CDLL(K.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", K.LIB_PATH], capture_output=True, text=True)
    exported = set(re.findall(r"\bT (kv_attn_\w+)", out.stdout))
    assert exported == set(declared)


def test_struct_layout_matches_the_header():
    """Compile a probe against the header and compare every offset with the ctypes mirror."""
    fields = {"kv_attn_params": K.kv_attn_params, "kv_attn_plan": K.kv_attn_plan}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "kv_attn.h"', "int main(void){"]
    for sname, cls in fields.items():
        lines.append(f'printf("{sname} size %zu\\n", sizeof({sname}));')
        for fname, _ in cls._fields_:
            lines.append(f'printf("{sname} {fname} %zu\\n", offsetof({sname}, {fname}));')
    lines.append("return 0;}")
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "probe.c"), os.path.join(d, "probe")
        open(src, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    for line in out.splitlines():
        sname, what, value = line.split()
        cls = fields[sname]
        if what == "size":
            assert ctypes.sizeof(cls) == int(value), sname
        else:
            assert getattr(cls, what).offset == int(value), (sname, what)


def test_abi_version_and_status_strings():
    assert K.kv_attn_abi_version() == 5
    for code in range(9):
        s = K.kv_attn_status_string(code)
        assert s and s != "unknown status"
    assert K.kv_attn_status_string(99) == "unknown status"


def _params(**kw):
    return K.make_params(**C.params_kwargs(**kw))


@pytest.mark.parametrize("kw,status", C.INVALID_PARAM_CASES)
def test_get_plan_rejects_invalid_params(kw, status):
    p = _params(**kw)
    with pytest.raises(K.KvAttnError) as e:
        K.kv_attn_get_plan(p, 256)
    assert e.value.status == getattr(K, status)


@pytest.mark.parametrize("field,value", [("window", -1), ("num_queries", -1)])
def test_get_plan_rejects_raw_field_values(field, value):
    """Fields the binding never sets this way are still checked by the library."""
    p = _params()
    setattr(p, field, value)
    with pytest.raises(K.KvAttnError) as e:
        K.kv_attn_get_plan(p, 256)
    assert e.value.status == K.KV_ATTN_ERR_VALUE


@pytest.mark.parametrize("kw", [
    dict(num_queries=17),                                   # more than 16 query tokens
    dict(num_queries=4, q_dtype=K.KV_ATTN_F32),             # rows mode is bf16 only
    dict(num_queries=4, kv_dtype=K.KV_ATTN_F32, k_strides=(8 * 16 * 128, 128, 16 * 128)),
    dict(num_queries=9),                                    # 9 tokens x group 4 = 36 rows > 32
    dict(num_queries=3, num_q_heads=8 * 16),                # 3 x 16 = 48 rows > 32
])
def test_unsupported_query_token_counts(kw):
    p = _params(**kw)
    with pytest.raises(K.KvAttnError) as e:
        K.kv_attn_get_plan(p, 256)
    assert e.value.status == K.KV_ATTN_ERR_UNSUPPORTED


@pytest.mark.parametrize("nq,hq,hkv", [(2, 32, 8), (4, 32, 8), (8, 32, 8), (4, 64, 8), (16, 8, 8)])
def test_plan_with_several_query_tokens(nq, hq, hkv):
    """gamma query tokens: matrix-core variant, merge rows and workspace scale with gamma."""
    B, T = 4, 8192
    p = _params(batch=B, num_q_heads=hq, num_kv_heads=hkv, max_ctx_len=T,
                max_blocks_per_seq=T // 16, num_blocks=10**6, num_queries=nq)
    plan = K.kv_attn_get_plan(p, 256)
    one = K.kv_attn_get_plan(_params(batch=B, num_q_heads=hq, num_kv_heads=hkv, max_ctx_len=T,
                                     max_blocks_per_seq=T // 16, num_blocks=10**6), 256)
    assert plan["kernel_variant"] == 2
    S, L = plan["num_splits"], plan["split_len"]
    assert L % 16 == 0 and S * L >= T and (S - 1) * L < T
    assert L <= 8192 and one["split_len"] <= 8192   # splits of at most 512 tiles
    # two row blocks keep one tile in flight per wave: about two workgroups per CU
    per_cu = 2 if nq * (hq // hkv) > 16 else 1
    # one row block, few units and >= 1024 tiles: each wave streams a split of its own KV head
    wh = per_cu == 1 and T // 16 >= 1024
    assert plan["wave_heads"] == int(wh)
    assert plan["grid_split"] == B * hkv * S // (4 if wh else 1) >= per_cu * 256
    if S > 1:
        assert plan["grid_merge"] == B * nq * hq
        assert plan["workspace_bytes"] >= B * nq * hq * S * (128 + 2) * 4


def test_binding_rejects_a_window_below_one():
    with pytest.raises(ValueError):
        _params(window=0)


@pytest.mark.parametrize("T,W,n", [(131072, 4096, 4), (131072, 1, 0), (131072, 4095, 17),
                                   (5000, 8192, 4), (100, 7, 200), (32768, 256, 0)])
def test_window_plan_sizes_the_grid_by_the_visited_tiles(T, W, n):
    """With a window the split grid covers the visited tiles of a sequence: at most the sink
    tiles plus the ceil(W/16) + 1 tiles the window touches, never more than the whole sequence."""
    p = _params(batch=4, num_q_heads=64, num_kv_heads=8, max_ctx_len=T,
                max_blocks_per_seq=(T + 15) // 16, num_blocks=10**6, window=W, num_sinks=n)
    plan = K.kv_attn_get_plan(p, 256)
    bound = min((T + 15) // 16, (min(n, T) + 15) // 16 + (W + 15) // 16 + 1)
    # The largest visited-tile count any length t <= T gives, enumerated directly.
    worst = 0
    for t in range(max(0, T - 64), T + 1):
        s_end, w0 = min(n, t), max(t - W, 0)
        tiles = {p // 16 for p in range(t) if p < s_end or p >= w0}
        worst = max(worst, len(tiles))
    assert worst <= bound
    S, L = plan["num_splits"], plan["split_len"]
    assert S * (L // 16) >= bound and (S - 1) * (L // 16) < bound


def test_plan_covers_every_tile_and_respects_bounds():
    for B, hkv, T in [(1, 8, 256), (8, 32, 4096), (64, 8, 8192), (128, 8, 32768), (4, 8, 131072),
                      (3, 2, 1), (2, 1, 17), (1, 1, 5000)]:
        for cus in (1, 80, 256, 304):
            p = _params(batch=B, num_q_heads=hkv * 2, num_kv_heads=hkv, max_ctx_len=T,
                        block_size=16, max_blocks_per_seq=(T + 15) // 16, num_blocks=10**6)
            plan = K.kv_attn_get_plan(p, cus)
            tiles = (T + 15) // 16
            S, L = plan["num_splits"], plan["split_len"]
            # head-major: each wave its own KV head with few units and >= 1024 tiles
            wh = (hkv % 4 == 0 and B * hkv * 2 < cus and tiles >= 1024
                  and tiles * (B * hkv // 4) >= 32 * cus)
            assert plan["wave_heads"] == int(wh), (B, hkv, T, cus)
            assert L % 16 == 0 and S >= 1
            assert S * L >= T and (S - 1) * L < T          # every position in exactly one split
            assert plan["grid_split"] == B * hkv * S // (4 if wh else 1)
            uo = 1 < S <= 256 and B * hkv // (4 if wh else 1) >= 4 * cus
            assert plan["unit_order"] == int(uo), (B, hkv, T, cus)
            if S > 1:
                # splits of >= 16 tiles when possible (>= 4 per wave either way)
                assert L // 16 >= min(4 if wh else 16, tiles)
                assert plan["workspace_bytes"] >= B * hkv * 2 * S * (128 + 2) * 4
                assert plan["grid_merge"] == B * hkv * 2
                _check_order_region(plan, B)
            else:
                assert plan["workspace_bytes"] == 0 and plan["grid_merge"] == 0
            # at most 256 tiles per split with many (sequence, KV head) units, 512 with few
            cap = 512 if B * hkv * 2 < cus else 256
            assert L // 16 <= cap or S == 4096


def test_random_plans_cover_the_visited_tiles_within_the_bounds():
    """Seeded sweep over shapes, windows, query tokens and CU counts: the splits cover exactly
    the tiles a sequence can visit, within the split-length bounds, and the workspace holds
    every split state."""
    for kw, cus, c in C.random_plan_cases():
        B, hkv, g, nq, T, W, n = (c[k] for k in ("B", "hkv", "g", "nq", "T", "W", "n"))
        plan = K.kv_attn_get_plan(K.make_params(**kw), cus)
        all_tiles = (T + 15) // 16
        bound = all_tiles if W == 0 else min(all_tiles, (min(n, T) + 15) // 16
                                              + (W + nq - 1 + 15) // 16 + 1)
        S, L = plan["num_splits"], plan["split_len"]
        label = (B, hkv, g, nq, T, W, n, cus, S, L)
        assert L % 16 == 0 and 1 <= S <= 4096, label
        assert S * (L // 16) >= bound and (S - 1) * (L // 16) < bound, label
        assert L // 16 <= 512 or S == 4096, label
        wh = (hkv % 4 == 0 and B * hkv * 2 < cus and nq * g <= 16 and bound >= 1024
              and bound * (B * hkv // 4) >= 32 * cus)
        assert plan["wave_heads"] == int(wh), label
        if S > 1:
            # at most one split per 16 visited tiles (per 4 when every wave streams a split)
            assert S <= -(-bound // (4 if wh else 16)), label
            rows = B * nq * hkv * g
            assert plan["grid_merge"] == rows
            assert plan["workspace_bytes"] >= rows * S * (128 + 2) * 4, label
            _check_order_region(plan, B)
        assert plan["grid_split"] == B * hkv * S // (4 if wh else 1), label
        # head_chunks (vector path, groups above 8 heads) keep the split-by-split order
        halves = plan["group_padded"] == 8 and g > 8
        uo = 1 < S <= 256 and not halves and B * hkv // (4 if wh else 1) >= 4 * cus
        assert plan["unit_order"] == int(uo), label


def _check_order_region(plan, B):
    """With unit order the workspace ends with the order list (B * S int32 pairs, 256-byte aligned,
    after the (m, l) array); without it there is none."""
    S = plan["num_splits"]
    if plan["unit_order"]:
        off = plan["order_offset"]
        assert off % 256 == 0 and off >= plan["ml_offset"]
        assert plan["workspace_bytes"] == off + B * S * 8
    else:
        assert plan["order_offset"] == 0


def test_unit_order_rule_and_override(monkeypatch):
    """C4 on 256 CUs (1024 split workgroups per split) takes the longest-first order; C3 (512),
    C5 and the unsplit C2 do not; KV_ATTN_UNIT_ORDER forces it either way where the shape allows
    it (S > 1, S <= 256, no halves)."""
    def plan(B, hq, hkv, T, cus=256, **kw):
        return K.kv_attn_get_plan(_params(batch=B, num_q_heads=hq, num_kv_heads=hkv, max_ctx_len=T,
                                          max_blocks_per_seq=(T + 15) // 16, num_blocks=10**6, **kw), cus)
    c4 = plan(128, 32, 8, 32768)
    assert c4["unit_order"] == 1 and c4["num_splits"] == 8
    assert c4["order_offset"] % 256 == 0 and c4["workspace_bytes"] == c4["order_offset"] + 128 * 8 * 8
    assert plan(64, 32, 8, 8192)["unit_order"] == 0          # C3: 512 units, two per CU
    assert plan(4, 64, 8, 131072)["unit_order"] == 0         # C5
    assert plan(8, 32, 32, 4096)["unit_order"] == 0          # C2: one split
    assert plan(128, 32, 8, 32768, cus=257)["unit_order"] == 0
    assert plan(128, 32, 8, 32768, cus=256, num_splits=300)["unit_order"] == 0   # S > 256
    monkeypatch.setenv("KV_ATTN_UNIT_ORDER", "0")
    off = plan(128, 32, 8, 32768)
    assert off["unit_order"] == 0 and off["order_offset"] == 0
    assert off["workspace_bytes"] <= c4["order_offset"]
    monkeypatch.setenv("KV_ATTN_UNIT_ORDER", "1")
    assert plan(64, 32, 8, 8192)["unit_order"] == 1
    assert plan(2, 8, 8, 700, num_splits=3)["unit_order"] == 1
    assert plan(2, 8, 8, 700, num_splits=1)["unit_order"] == 0          # one split: nothing to order
    assert plan(2, 8, 8, 16384, num_splits=600)["unit_order"] == 0      # S = 512 > 256
    halves = plan(2, 32, 2, 700, num_splits=3, q_dtype=0, kv_dtype=0)   # fp32, group 16: halves
    assert halves["unit_order"] == 0


def test_plan_for_the_five_workloads():
    """Launch geometry of C1-C5 on a 256-CU device (what the bench times)."""
    want = {  # (B, h_q, h_kv, T) -> (S, split_len)
        (1, 8, 8, 256): (1, 256),
        (8, 32, 32, 4096): (1, 4096),
        (64, 32, 8, 8192): (2, 4096),
        (128, 32, 8, 32768): (8, 4096),
        (4, 64, 8, 131072): (32, 4096),    # few units: each wave streams a split of its own KV head
    }
    for (B, hq, hkv, T), (S, L) in want.items():
        p = _params(batch=B, num_q_heads=hq, num_kv_heads=hkv, max_ctx_len=T,
                    max_blocks_per_seq=(T + 15) // 16, num_blocks=10**6)
        plan = K.kv_attn_get_plan(p, 256)
        assert (plan["num_splits"], plan["split_len"]) == (S, L)
        # groups of 4 or more run P.V on the matrix cores too (rows mode)
        assert plan["kernel_variant"] == (2 if hq // hkv >= 4 else 1)


_token_major = C.token_major


def test_token_major_plan_gives_each_wave_its_own_kv_head():
    """Token-major caches with h_kv a multiple of 4 and fewer than 4 units per CU: four KV heads
    per split workgroup, one per wave, each wave streaming a whole split."""
    p = _params(batch=4, num_q_heads=64, num_kv_heads=8, max_ctx_len=131072,
                max_blocks_per_seq=8192, num_blocks=10**6, **_token_major(8))
    plan = K.kv_attn_get_plan(p, 256)
    assert plan["wave_heads"] == 1
    assert (plan["num_splits"], plan["split_len"]) == (32, 4096)   # 8 workgroups per split
    assert plan["grid_split"] == 4 * 2 * 32 and plan["grid_merge"] == 4 * 64
    for (B, hq, hkv, T), S in {(8, 32, 32, 4096): 4, (64, 32, 8, 8192): 2}.items():
        p = _params(batch=B, num_q_heads=hq, num_kv_heads=hkv, max_ctx_len=T,
                    max_blocks_per_seq=T // 16, num_blocks=10**6, **_token_major(hkv))
        plan = K.kv_attn_get_plan(p, 256)
        assert plan["wave_heads"] == 1 and plan["num_splits"] == S, (B, hkv)
    # 4 * num_cus units or more (C4's 1024) keep one KV head per workgroup
    p = _params(batch=128, num_q_heads=32, num_kv_heads=8, max_ctx_len=32768,
                max_blocks_per_seq=2048, num_blocks=10**6, **_token_major(8))
    assert K.kv_attn_get_plan(p, 256)["wave_heads"] == 0
    assert K.kv_attn_get_plan(p, 257)["wave_heads"] == 1
    # head-major: only with few units, one row block and >= 1024 tiles
    hm = dict(batch=4, num_q_heads=64, num_kv_heads=8, max_ctx_len=131072,
              max_blocks_per_seq=8192, num_blocks=10**6)
    assert K.kv_attn_get_plan(_params(**hm), 256)["wave_heads"] == 1
    two_blocks = K.kv_attn_get_plan(_params(**hm, num_queries=4), 256)
    assert two_blocks["wave_heads"] == 0 and two_blocks["num_splits"] == 16
    assert K.kv_attn_get_plan(_params(**dict(hm, max_ctx_len=16368)), 256)["wave_heads"] == 0
    assert K.kv_attn_get_plan(_params(**dict(hm, max_ctx_len=16369)), 256)["wave_heads"] == 1
    assert K.kv_attn_get_plan(_params(**hm, window=4096, num_sinks=4), 256)["wave_heads"] == 0
    # too little work per wave on a full device (a 4096-position window, 256 positions)
    assert K.kv_attn_get_plan(_params(**hm, window=4096, num_sinks=4, **_token_major(8)),
                              256)["wave_heads"] == 0
    assert K.kv_attn_get_plan(_params(batch=1, num_q_heads=8, num_kv_heads=8, max_ctx_len=256,
                                      max_blocks_per_seq=16, **_token_major(8)), 256)["wave_heads"] == 0
    many = dict(batch=8, num_q_heads=32, num_kv_heads=32, max_ctx_len=4096, max_blocks_per_seq=256)
    assert K.kv_attn_get_plan(_params(**many), 256)["wave_heads"] == 0
    assert K.kv_attn_get_plan(_params(**many, **_token_major(32)), 256)["wave_heads"] == 1
    # h_kv not a multiple of 4, or the vector path's halves: one KV head per workgroup
    assert K.kv_attn_get_plan(_params(num_q_heads=4, num_kv_heads=2, **_token_major(2)), 256)["wave_heads"] == 0
    p = _params(num_q_heads=8 * 16, q_dtype=K.KV_ATTN_F32, **_token_major(8))
    assert K.kv_attn_get_plan(p, 256)["wave_heads"] == 0
    # a caller-given split count is kept
    p = _params(num_splits=3, max_ctx_len=20000, max_blocks_per_seq=1250, num_blocks=10**6,
                **_token_major(8))
    plan = K.kv_attn_get_plan(p, 256)
    assert plan["wave_heads"] == 1 and plan["num_splits"] == 3 and plan["grid_split"] == 4 * 2 * 3


def test_random_token_major_plans_cover_the_tiles():
    for kw, cus, c in C.random_token_major_cases():
        B, hkv, g, T, W = (c[k] for k in ("B", "hkv", "g", "T", "W"))
        plan = K.kv_attn_get_plan(K.make_params(**kw), cus)
        all_tiles = (T + 15) // 16
        bound = all_tiles if W == 0 else min(all_tiles, 1 + (W + 15) // 16 + 1)
        S, L = plan["num_splits"], plan["split_len"]
        label = (B, hkv, g, T, W, cus, S, L)
        wh = B * hkv < 4 * cus and bound * (B * hkv // 4) >= 32 * cus
        assert plan["wave_heads"] == int(wh), label
        assert L % 16 == 0 and 1 <= S <= 4096, label
        assert S * (L // 16) >= bound and (S - 1) * (L // 16) < bound, label
        assert L // 16 <= 512 or S == 4096, label
        assert plan["grid_split"] == (B * (hkv // 4) if wh else B * hkv) * S, label
        if S > 1:
            assert plan["workspace_bytes"] >= B * hkv * g * S * (128 + 2) * 4, label


def test_explicit_split_count_and_variant_selection():
    p = _params(num_splits=3)
    plan = K.kv_attn_get_plan(p, 256)
    assert plan["num_splits"] == 3 and plan["split_len"] == 336
    p = _params(q_dtype=K.KV_ATTN_F32)
    assert K.kv_attn_get_plan(p, 256)["kernel_variant"] == 0
    p = _params(num_q_heads=8 * 3)
    assert K.kv_attn_get_plan(p, 256)["group_padded"] == 4
    assert K.kv_attn_get_plan(p, 256)["kernel_variant"] == 1
    for g in (4, 5, 16):
        assert K.kv_attn_get_plan(_params(num_q_heads=8 * g), 256)["kernel_variant"] == 2, g
    p = _params(num_q_heads=8 * 8, q_dtype=K.KV_ATTN_F32, kv_dtype=K.KV_ATTN_F32)
    assert K.kv_attn_get_plan(p, 256)["kernel_variant"] == 0
    # the vector path serves a group above 8 heads with two workgroups of up to 8 heads each
    for g in (9, 16):
        for qd, kd in ((K.KV_ATTN_F32, K.KV_ATTN_F32), (K.KV_ATTN_BF16, K.KV_ATTN_F32)):
            plan = K.kv_attn_get_plan(_params(num_q_heads=8 * g, q_dtype=qd, kv_dtype=kd), 256)
            assert plan["kernel_variant"] == 0 and plan["group_padded"] == 8
            assert plan["grid_split"] == 2 * 4 * 8 * plan["num_splits"]


def _decode_raw(p, q=16, k=16, v=16, bt=16, ctx=16, out=16, ws=None, ws_bytes=0):
    lib = K._lib
    return lib.kv_attn_decode(q, k, v, bt, ctx, out, ctypes.byref(p), ws, ws_bytes, None)


def test_decode_null_pointers_fail_before_any_hip_call():
    p = _params()
    assert _decode_raw(p, q=None) == K.KV_ATTN_ERR_NULL
    assert _decode_raw(p, ctx=None) == K.KV_ATTN_ERR_NULL
    assert _decode_raw(p, out=None) == K.KV_ATTN_ERR_NULL
    assert K._lib.kv_attn_decode(16, 16, 16, 16, 16, 16, None, None, 0, None) == K.KV_ATTN_ERR_NULL


def test_decode_layout_errors_fail_before_any_hip_call():
    for kw in C.INVALID_LAYOUT_CASES:
        assert _decode_raw(_params(**kw)) == K.KV_ATTN_ERR_SHAPE, kw
    assert _decode_raw(_params(block_size=500), bt=None) == K.KV_ATTN_ERR_SHAPE  # capacity < max ctx
    assert _decode_raw(_params(block_size=1000, num_blocks=3), bt=None) == K.KV_ATTN_ERR_SHAPE
    assert _decode_raw(_params(), q=8) == K.KV_ATTN_ERR_UNSUPPORTED              # misaligned
    assert _decode_raw(_params(head_dim=32)) == K.KV_ATTN_ERR_UNSUPPORTED


def test_simulated_hip_failure(monkeypatch):
    monkeypatch.setenv("KV_ATTN_FAULT", "query")
    assert _decode_raw(_params()) == K.KV_ATTN_ERR_HIP
    plan = K.kv_attn_plan()
    assert K._lib.kv_attn_get_plan(ctypes.byref(_params()), 0, ctypes.byref(plan)) == K.KV_ATTN_ERR_HIP
    assert K.kv_attn_workspace_size(_params()) == 0


def test_merge_argument_errors():
    lib = K._lib
    assert lib.kv_attn_merge(None, 16, None, 16, 4, 2, 128, None) == K.KV_ATTN_ERR_NULL
    assert lib.kv_attn_merge(16, 16, None, 16, 0, 2, 128, None) == K.KV_ATTN_ERR_SHAPE
    assert lib.kv_attn_merge(16, 16, None, 16, 4, 0, 128, None) == K.KV_ATTN_ERR_SHAPE
    assert lib.kv_attn_merge(16, 16, None, 16, 4, 2, 100, None) == K.KV_ATTN_ERR_UNSUPPORTED
    assert lib.kv_attn_merge(16, 16, None, 16, 4, 4097, 128, None) == K.KV_ATTN_ERR_UNSUPPORTED


def test_host_validator():
    p = _params(batch=3, max_ctx_len=40, max_blocks_per_seq=3, num_blocks=10)
    ctx = torch.tensor([40, 1, 0], dtype=torch.int32)
    bt = torch.tensor([[0, 1, 2], [9, -5, -5], [-1, -1, -1]], dtype=torch.int32)
    assert K.kv_attn_validate_host(bt, ctx, p) == K.KV_ATTN_OK
    bad = bt.clone()
    bad[0, 2] = 10
    assert K.kv_attn_validate_host(bad, ctx, p) == K.KV_ATTN_ERR_TABLE
    bad = bt.clone()
    bad[1, 0] = -1
    assert K.kv_attn_validate_host(bad, ctx, p) == K.KV_ATTN_ERR_TABLE
    assert K.kv_attn_validate_host(bt, torch.tensor([41, 1, 0], dtype=torch.int32), p) == K.KV_ATTN_ERR_TABLE
    assert K.kv_attn_validate_host(bt, torch.tensor([3, -1, 0], dtype=torch.int32), p) == K.KV_ATTN_ERR_TABLE
    pc = _params(batch=3, max_ctx_len=40, block_size=40, num_blocks=3)
    assert K.kv_attn_validate_host(None, ctx, pc) == K.KV_ATTN_OK


def test_binding_rejects_tensors_too_small_for_the_strides():
    k = torch.zeros(2, 2, 8, 64, dtype=torch.bfloat16)  # contiguous head major, capacity 8
    strides = (2 * 8 * 64, 64, 8 * 64)
    K._check_extent(k, strides, 2, 8, 2, 64, "k_cache")  # exactly the tensor: accepted
    with pytest.raises(ValueError, match="strides address"):
        K._check_extent(k, strides, 2, 9, 2, 64, "k_cache")  # a ninth slot per block
    with pytest.raises(ValueError, match="strides address"):
        K._check_extent(k[1:], strides, 2, 8, 2, 64, "k_cache")  # a view that starts later


def test_binding_refuses_host_tensors_before_any_library_call():
    """Host tensors would reach the kernels as host addresses: every entry of the binding that
    takes tensors refuses them first."""
    from kv_cache_decode_split_amd import kv_evict as E
    q = torch.zeros(2, 4, 64, dtype=torch.bfloat16)
    out = torch.zeros(2, 4, 64, dtype=torch.float32)
    k = torch.zeros(2, 2, 8, 64, dtype=torch.bfloat16)
    ctx = torch.tensor([8, 8], dtype=torch.int32)
    strides = (2 * 8 * 64, 64, 8 * 64)
    with pytest.raises(ValueError, match="device"):
        K.kv_attn_decode(q, k, k, None, ctx, out, num_kv_heads=2, k_strides=strides,
                         v_strides=strides, block_size=8, num_blocks=2, max_ctx_len=8)
    rows = torch.zeros(2, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device"):
        K.kv_attn_append(rows, rows, k, k, None, torch.zeros(2, dtype=torch.int32), num_kv_heads=2,
                         k_strides=strides, v_strides=strides, block_size=8, num_blocks=2)
    with pytest.raises(ValueError, match="device"):
        K.kv_attn_merge(torch.zeros(3, 2, 64), torch.zeros(3, 2, 2), None, torch.zeros(3, 64))
    with pytest.raises(ValueError):
        E.kv_evict_select(torch.zeros(2, 2, 16), 8)
    with pytest.raises(ValueError):
        K.kv_attn_read_probe(torch.zeros(1024, dtype=torch.uint8), torch.zeros(1, dtype=torch.int32))


def test_append_argument_errors_fail_before_any_hip_call():
    lib = K._lib
    p = _params()
    assert lib.kv_attn_append(None, 16, 16, 16, 16, 16, ctypes.byref(p), None) == K.KV_ATTN_ERR_NULL
    assert lib.kv_attn_append(16, 16, 16, 16, 16, None, ctypes.byref(p), None) == K.KV_ATTN_ERR_NULL
    assert lib.kv_attn_append(16, 16, 16, 16, 16, 16, None, None) == K.KV_ATTN_ERR_NULL
    assert lib.kv_attn_append(8, 16, 16, 16, 16, 16, ctypes.byref(p), None) == K.KV_ATTN_ERR_UNSUPPORTED
    bad = _params(block_size=24)
    assert lib.kv_attn_append(16, 16, 16, 16, 16, 16, ctypes.byref(bad), None) == K.KV_ATTN_ERR_SHAPE
    # append + decode: a missing new row fails before anything else
    assert lib.kv_attn_append_decode(16, None, 16, 16, 16, 16, 16, 16, ctypes.byref(p), None, 0,
                                     None) == K.KV_ATTN_ERR_NULL
    assert lib.kv_attn_append_decode(16, 8, 16, 16, 16, 16, 16, 16, ctypes.byref(p), None, 0,
                                     None) == K.KV_ATTN_ERR_UNSUPPORTED


def test_read_probe_rejects_bad_arguments_before_any_hip_call():
    lib = K._lib
    assert lib.kv_attn_read_probe(None, 1 << 20, 16, None) == K.KV_ATTN_ERR_NULL
    assert lib.kv_attn_read_probe(16, 1 << 20, None, None) == K.KV_ATTN_ERR_NULL
    assert lib.kv_attn_read_probe(16, 0, 16, None) == K.KV_ATTN_ERR_UNSUPPORTED
    assert lib.kv_attn_read_probe(16, 1000, 16, None) == K.KV_ATTN_ERR_UNSUPPORTED   # not x16
    assert lib.kv_attn_read_probe(8, 1 << 20, 16, None) == K.KV_ATTN_ERR_UNSUPPORTED  # misaligned
