"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same inputs.

Small cases span several tiles, several splits and a ragged last tile and are compared element
by element; the five workloads at full size (in the launch configuration the bench times) are
compared on every output row as well, the oracle running over chunks of sequences. Tolerance:
max abs error <= 5e-3 and max abs error / max |ref| <= 1e-2 on the fp32 output.
"""

import random

import pytest
import torch

from kv_cache_decode_split_amd import workloads as W
from tests.gpu_helpers import (announce, check_close, loaded_native_libraries, oracle_full,
                               oracle_rows, require_gpu, run, select_rows)

pytestmark = pytest.mark.gpu


def test_native_library_is_the_one_running():
    require_gpu()
    libs = loaded_native_libraries()
    assert libs and all(p.endswith("kv_cache_decode_split_amd/libkvattn.so") for p in libs), libs


SMALL = [
    ("C1", dict()),
    ("C1", dict(num_splits=4)),
    ("C2", dict(batch=2, ctx=(700, 700))),
    ("C2", dict(batch=2, ctx=(700, 333), capacity=720, layout="token_major")),
    ("C3", dict(batch=3, ctx=(1000,) * 3)),
    ("C4", dict(batch=6, ctx=("uniform", 1, 700))),
    ("C4", dict(batch=5, ctx=("uniform", 1, 300), layout="token_major", extra_blocks=7)),
    ("C5", dict(batch=2, ctx=(3000, 2999))),
    ("C5", dict(batch=3, ctx=(3000, 1, 2999), block_order="sequential")),
    # vector path above 8 heads per KV head: two workgroups serve the halves of the group
    ("C1", dict(batch=2, ctx=(700, 333), head_dim=128, num_q_heads=32, num_kv_heads=2)),
    ("C4", dict(batch=3, ctx=(900, 1, 450), num_q_heads=96, num_kv_heads=8, q_dtype="f32")),
    ("C4", dict(batch=6, ctx=("uniform", 1, 700), block_order="sequential", num_kv_heads=16,
                num_q_heads=32)),
    # token-major caches with h_kv a multiple of 4 (rows mode, MFMA scores with VALU P.V, the
    # vector path, and a contiguous cache)
    ("C5", dict(batch=2, ctx=(3000, 2999), layout="token_major")),
    ("C2", dict(batch=2, ctx=(1500, 33), num_q_heads=8, num_kv_heads=8, layout="token_major")),
    ("C1", dict(batch=3, ctx=(700, 1, 333), head_dim=128, num_q_heads=32, num_kv_heads=4,
                q_dtype="f32", layout="token_major")),
    ("C3", dict(batch=3, ctx=(1000, 17, 999), capacity=1000, layout="token_major")),
    # the shapes of two kernel variants that once returned wrong values (both then compiled to
    # heavily spilling vector kernels): fp32 q with bf16 KV, g = 16, d = 64; fp32 q and KV,
    # g = 16, d = 128 (also a score-export case)
    ("C1", dict(batch=3, ctx=(700, 1, 333), head_dim=64, num_q_heads=32, num_kv_heads=2,
                kv_dtype="bf16")),
    ("C1", dict(batch=3, ctx=(900, 17, 450), head_dim=128, num_q_heads=32, num_kv_heads=2)),
]


@pytest.mark.parametrize("name,over", SMALL, ids=[f"{n}-{i}" for i, (n, _) in enumerate(SMALL)])
@pytest.mark.parametrize("num_splits", [0, 1, 5])
def test_small_workloads_match_oracle(name, over, num_splits):
    require_gpu()
    kw = dict(over)
    forced = kw.pop("num_splits", None)
    spec = W.preset(name, **kw)
    announce(f"small {name} {kw} num_splits={forced or num_splits}")
    w = W.make_workload(spec, device="cuda")
    out = run(w, num_splits=forced if forced is not None else num_splits)
    check_close(out.cpu().numpy(), oracle_full(w), f"{name} {kw} S={num_splits}")


def _random_specs(n, seed=7):
    rnd = random.Random(seed)
    specs = []
    for i in range(n):
        d = rnd.choice([64, 128])
        g = rnd.choice([1, 2, 3, 4, 5, 8, 16])
        hkv = rnd.choice([1, 2, 3])
        B = rnd.randint(1, 4)
        paged = rnd.random() < 0.5
        lens = tuple(rnd.randint(1, 2500) for _ in range(B))
        if rnd.random() < 0.2:
            lens = tuple(rnd.randint(1, 40) for _ in range(B))
        qd, kd = rnd.choice([("bf16", "bf16"), ("bf16", "bf16"), ("f32", "f32"), ("f32", "bf16"),
                             ("bf16", "f32")])
        specs.append(dict(
            spec=W.WorkloadSpec(
                name=f"rand{i}", batch=B, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d, ctx=lens,
                paged=paged, block_size=rnd.choice([16, 32, 64]) if paged else 16, kv_dtype=kd,
                q_dtype=qd, q_std=rnd.choice([1.0, 2.0, 4.0]), num_sinks=rnd.choice([0, 0, 4]),
                layout=rnd.choice(["head_major", "token_major"]), seed=5000 + i,
                extra_blocks=rnd.randint(1, 4),
                capacity=None if paged else max(lens) + rnd.choice([0, 0, 5])),
            num_splits=rnd.choice([0, 0, 1, 2, 7])))
    return specs


RANDOM = _random_specs(40)


def _random_wave_head_specs(n, seed=8):
    """Token-major caches with h_kv in {4, 8, 12}, each wave of a split workgroup serving its own
    KV head (forced: the planner picks that for long sequences only)."""
    rnd = random.Random(seed)
    specs = []
    for i in range(n):
        hkv = rnd.choice([4, 8, 12])
        g = rnd.choice([1, 2, 4, 8])
        B = rnd.randint(1, 3)
        paged = rnd.random() < 0.7
        lens = tuple(rnd.randint(1, 3000) for _ in range(B))
        qd, kd = rnd.choice([("bf16", "bf16"), ("bf16", "bf16"), ("f32", "f32"), ("f32", "bf16")])
        specs.append(dict(
            spec=W.WorkloadSpec(
                name=f"wh{i}", batch=B, num_q_heads=g * hkv, num_kv_heads=hkv,
                head_dim=rnd.choice([64, 128]), ctx=lens, paged=paged,
                block_size=rnd.choice([16, 32]) if paged else 16, kv_dtype=kd, q_dtype=qd,
                num_sinks=rnd.choice([0, 4]), layout="token_major", seed=5600 + i,
                extra_blocks=rnd.randint(1, 4), capacity=None if paged else max(lens)),
            num_splits=rnd.choice([0, 0, 1, 3])))
    return specs


RANDOM_WAVE_HEADS = _random_wave_head_specs(12)


@pytest.mark.parametrize("case", RANDOM_WAVE_HEADS, ids=[c["spec"].name for c in RANDOM_WAVE_HEADS])
def test_token_major_wave_heads_match_oracle(case, monkeypatch):
    K = require_gpu()
    monkeypatch.setenv("KV_ATTN_WAVE_HEADS", "1")
    spec = case["spec"]
    announce(f"wave heads {spec}")
    w = W.make_workload(spec, device="cuda")
    out = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")
    assert K.decode_call_for(w, out, num_splits=case["num_splits"]).plan()["wave_heads"] == 1
    got = run(w, num_splits=case["num_splits"])
    check_close(got.cpu().numpy(), oracle_full(w), spec.name)


@pytest.mark.parametrize("case", RANDOM, ids=[c["spec"].name for c in RANDOM])
def test_random_shapes_match_oracle(case):
    require_gpu()
    spec = case["spec"]
    announce(f"random {spec}")
    w = W.make_workload(spec, device="cuda")
    out = run(w, num_splits=case["num_splits"])
    check_close(out.cpu().numpy(), oracle_full(w), spec.name)


def test_explicit_scale_matches_oracle():
    require_gpu()
    w = W.make_workload(W.preset("C3", batch=2, ctx=(500, 77)), device="cuda")
    out = run(w, scale=0.05)
    check_close(out.cpu().numpy(), oracle_full(w, scale=0.05), "scale=0.05")


FULL = ["C1", "C2", "C3", "C4", "C5", "C5-sequential", "C5-token_major", "C4-kv4"]

# Host bytes of bf16 K/V copied per oracle chunk (the oracle widens one (sequence, KV head) at a
# time, so its own memory stays far below this).
CHUNK_BYTES = 1 << 30


def _sequence_chunks(w: W.Workload, limit: int = CHUNK_BYTES):
    """Consecutive runs of sequences whose cached K/V together stay under ``limit`` bytes."""
    elem = w.k_cache.element_size()
    per_pos = 2 * w.spec.num_kv_heads * w.spec.head_dim * elem
    chunks, cur, size = [], [], 0
    for b, t in enumerate(w.ctx_lens.cpu().tolist()):
        if cur and size + t * per_pos > limit:
            chunks.append(cur)
            cur, size = [], 0
        cur.append(b)
        size += t * per_pos
    if cur:
        chunks.append(cur)
    return chunks


@pytest.mark.parametrize("name", FULL)
def test_full_size_workloads_on_every_row(name):
    """The bench's launch configuration (auto split plan) at full size; every output row of the
    batch is compared with the oracle, which runs over consecutive chunks of sequences.

    C2 is one of its 32 layers (layer 0). C5-sequential deals the blocks to the sequences in
    physical order; C5-token_major stores the cache token-major (each wave of a workgroup then
    serves its own KV head); C4-kv4 is C4's ragged batch with 4 KV heads (group 4), whose split
    workgroups are dealt to the XCDs with the per-split sequence shift.
    """
    require_gpu()
    announce(f"full {name}")
    base, _, variant = name.partition("-")
    if variant == "token_major":
        spec = W.preset(base, layout="token_major")
    elif variant == "kv4":
        spec = W.preset(base, num_q_heads=16, num_kv_heads=4)
    else:
        spec = W.preset(base, block_order=variant) if variant else W.PRESETS[base]
    w = W.make_workload(spec, device="cuda")
    try:
        out = run(w)
        rows = 0
        for seqs in _sequence_chunks(w):
            ref = oracle_rows(w, seqs)
            check_close(select_rows(out, w, seqs), ref, f"full {name} seqs {seqs[0]}..{seqs[-1]}")
            rows += ref.shape[0] * ref.shape[1]
        assert rows == out.shape[0] * out.shape[1]
    finally:
        del w
        torch.cuda.empty_cache()
