"""The library's host layer under the address and undefined-behaviour sanitizers (CPU only).

``kv_attn_plan.cpp`` (argument validation, split planning, the host-side table validator and the
status strings) is compiled with g++ and ``-fsanitize=address,undefined`` together with a small
driver (``tests/native/plan_harness.cpp``; no HIP, nothing runs on a device) and fed the seeded
planning sweeps, the invalid-parameter and layout cases and the validator cases of the ABI
tests. The run must end cleanly with no sanitizer report, and every plan must equal the one the
built library returns for the same problem.
"""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from tests import plan_cases as C

K = pytest.importorskip("kv_cache_decode_split_amd.kv_attn",
                        reason="libkvattn.so not built (run python -m kv_cache_decode_split_amd.build)")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_decode_split_amd", "csrc")
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    gxx = shutil.which(os.environ.get("CXX", "g++"))
    if gxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("sanitize") / "plan_harness")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", *SANITIZE,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "native", "plan_harness.cpp"),
           os.path.join(CSRC, "kv_attn_plan.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def _fields(kw: dict) -> str:
    p = K.make_params(**kw)
    vals = []
    for name, _ in K.kv_attn_params._fields_:
        v = getattr(p, name)
        vals.append(repr(float(v)) if name == "scale" else str(int(v)))
    return " ".join(vals)


def _run(exe: str, text: str) -> list:
    env = dict(os.environ)
    # The sanitizer runtime need not come first among preloaded libraries, leaks are reported,
    # and the first report ends the run with a non-zero status.
    env["ASAN_OPTIONS"] = "verify_asan_link_order=0:detect_leaks=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    proc = subprocess.run([exe], input=text, capture_output=True, text=True, env=env, timeout=300)
    assert "runtime error" not in proc.stderr and "Sanitizer" not in proc.stderr, proc.stderr[-4000:]
    assert proc.returncode == 0, proc.stderr[-4000:]
    return proc.stdout.splitlines()


def _library_plan(kw: dict, cus: int):
    """(status, fields) the built library gives; fields compare with the harness's output."""
    try:
        plan = K.kv_attn_get_plan(K.make_params(**kw), cus)
    except K.KvAttnError as e:
        return e.status, None
    return K.KV_ATTN_OK, (plan["num_splits"], plan["split_len"] // 16, plan["grid_split"],
                          plan["grid_merge"], plan["kernel_variant"], plan["group_padded"],
                          plan["wave_heads"], plan["workspace_bytes"])


def test_planning_and_validation_run_clean_under_sanitizers(harness):
    cases = [(kw, cus) for kw, cus, _ in C.random_plan_cases()]
    cases += [(kw, cus) for kw, cus, _ in C.random_token_major_cases()]
    cases += [(C.params_kwargs(**kw), 256) for kw, _ in C.INVALID_PARAM_CASES]
    cases += [(C.params_kwargs(**kw), 256) for kw in C.INVALID_LAYOUT_CASES]
    lines = [f"P {_fields(kw)} {cus} 1" for kw, cus in cases]
    # contiguous caches: the slot capacity must hold max_ctx_len and every sequence
    lines += [f"P {_fields(C.params_kwargs(block_size=bs, num_blocks=nb))} 256 0"
              for bs, nb in ((1000, 4), (999, 4), (1000, 3))]
    # the host validator: good tables, entries out of range, lengths out of range, contiguous
    vkw = C.params_kwargs(batch=3, max_ctx_len=40, max_blocks_per_seq=3, num_blocks=10)
    good = [0, 1, 2, 9, -5, -5, -1, -1, -1]
    validator = [
        ([40, 1, 0], good, K.KV_ATTN_OK),
        ([40, 1, 0], [0, 1, 10] + good[3:], K.KV_ATTN_ERR_TABLE),
        ([40, 1, 0], good[:3] + [-1] + good[4:], K.KV_ATTN_ERR_TABLE),
        ([41, 1, 0], good, K.KV_ATTN_ERR_TABLE),
        ([3, -1, 0], good, K.KV_ATTN_ERR_TABLE),
        ([40, 40, 40], list(range(9)), K.KV_ATTN_OK),
    ]
    for ctx, table, _ in validator:
        lines.append(f"V {_fields(vkw)} 1 {' '.join(map(str, ctx))} {' '.join(map(str, table))}")
    ckw = C.params_kwargs(batch=3, max_ctx_len=40, block_size=40, num_blocks=3)
    lines.append(f"V {_fields(ckw)} 0 40 1 0")
    lines.append(f"V {_fields(C.params_kwargs(batch=0))} 0")
    lines += [f"S {code}" for code in range(-1, 10)]

    out = _run(harness, "\n".join(lines) + "\n")
    assert len(out) == len(lines)

    plans = out[:len(cases) + 3]
    n_layout = len(C.INVALID_LAYOUT_CASES)
    for i, ((kw, cus), got) in enumerate(zip(cases, plans[:len(cases)])):
        parts = [int(x) for x in got.split()[1:]]
        status, fields = _library_plan(kw, cus)
        assert parts[1] == status, (kw, cus, got)
        if status == K.KV_ATTN_OK:
            assert tuple(parts[2:]) == fields, (kw, cus, got, fields)
            if i < len(cases) - n_layout:   # the sweeps are valid paged layouts
                assert parts[0] == K.KV_ATTN_OK, (kw, got)
    invalid_layout = plans[len(cases) - n_layout:len(cases)]
    assert all(int(x.split()[1]) == K.KV_ATTN_ERR_SHAPE for x in invalid_layout), invalid_layout
    contiguous = [int(x.split()[1]) for x in plans[len(cases):]]
    assert contiguous == [K.KV_ATTN_OK, K.KV_ATTN_ERR_SHAPE, K.KV_ATTN_ERR_SHAPE], contiguous

    rest = out[len(cases) + 3:]
    want = [w for _, _, w in validator] + [K.KV_ATTN_OK, K.KV_ATTN_ERR_SHAPE]
    assert [int(x.split()[1]) for x in rest[:len(want)]] == want
    strings = [x[2:] for x in rest[len(want):]]
    assert strings == [K.kv_attn_status_string(code) for code in range(-1, 10)]
