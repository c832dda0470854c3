"""GPU parity of sliding-window / attention-sink decode against the fp64 oracle.

With a window W and n sinks a sequence of length T attends to its first min(n, T) and its last
min(W, T) positions (each once); every other position of the cache is NaN-poisoned by the
workload generator, so an output that is finite and matches the oracle also shows that the
kernel never read a position outside the two ranges. Tolerance as for the other parity tests.
"""

import random

import numpy as np
import pytest
import torch

from kv_cache_decode_split_amd import workloads as W
from tests.gpu_helpers import (announce, check_close, oracle_full, oracle_rows, require_gpu, run,
                               select_rows)

pytestmark = pytest.mark.gpu


SMALL = [
    # (preset, overrides, window, sinks)
    ("C5", dict(batch=3, ctx=(3000, 2999, 700)), 1000, 4),        # gap between sinks and window
    ("C5", dict(batch=2, ctx=(1500, 33)), 17, 5),                  # edges inside tiles
    ("C5", dict(batch=2, ctx=(24, 40)), 10, 3),                    # sinks and window share a tile
    ("C5", dict(batch=2, ctx=(40, 300)), 30, 20),                  # sinks overlap the window
    ("C5", dict(batch=2, ctx=(300, 200)), 64, 500),                # every position is a sink
    ("C5", dict(batch=2, ctx=(2000, 1)), 1, 0),                    # window of one
    ("C4", dict(batch=6, ctx=("uniform", 1, 700), layout="token_major", extra_blocks=5), 100, 16),
    ("C4", dict(batch=4, ctx=("uniform", 200, 900), block_size=64), 256, 0),
    ("C3", dict(batch=3, ctx=(1000, 77, 300), capacity=1010), 300, 0),
    ("C2", dict(batch=2, ctx=(700, 333)), 5000, 0),                # window longer than T
    ("C1", dict(ctx=(256,)), 50, 2),                               # fp32 vector path
    ("C1", dict(batch=2, ctx=(256, 100), kv_dtype="bf16", head_dim=128), 33, 1),
    ("C5", dict(batch=2, ctx=(900, 901), num_q_heads=16 * 2, num_kv_heads=2, head_dim=64), 200, 4),
]


@pytest.mark.parametrize("name,over,window,sinks", SMALL,
                         ids=[f"{n}-{i}" for i, (n, *_) in enumerate(SMALL)])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_small_windowed_workloads_match_oracle(name, over, window, sinks, num_splits):
    require_gpu()
    spec = W.preset(name, window=window, num_sinks=sinks, **over)
    announce(f"window {name} {over} W={window} sinks={sinks} num_splits={num_splits}")
    w = W.make_workload(spec, device="cuda")
    out = run(w, num_splits=num_splits)
    check_close(out.cpu().numpy(), oracle_full(w), f"{name} W={window} n={sinks} S={num_splits}")


def _random_window_specs(n, seed=11):
    rnd = random.Random(seed)
    specs = []
    for i in range(n):
        d = rnd.choice([64, 128])
        g = rnd.choice([1, 2, 4, 5, 8, 16])
        hkv = rnd.choice([1, 2, 3])
        B = rnd.randint(1, 4)
        paged = rnd.random() < 0.6
        lens = tuple(rnd.randint(0 if rnd.random() < 0.1 else 1, 3000) for _ in range(B))
        if max(lens) == 0:
            lens = (1,) + lens[1:]
        qd, kd = rnd.choice([("bf16", "bf16"), ("bf16", "bf16"), ("f32", "f32"), ("f32", "bf16")])
        specs.append(dict(
            spec=W.WorkloadSpec(
                name=f"rwin{i}", batch=B, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d,
                ctx=lens, paged=paged, block_size=rnd.choice([16, 32, 128]) if paged else 16,
                kv_dtype=kd, q_dtype=qd, q_std=rnd.choice([1.0, 3.0]),
                num_sinks=rnd.choice([0, 1, 4, 16, 37]), window=rnd.choice([1, 15, 16, 100, 513, 2048]),
                layout=rnd.choice(["head_major", "token_major"]), seed=7000 + i,
                extra_blocks=rnd.randint(1, 3), capacity=None if paged else max(lens) + 3),
            num_splits=rnd.choice([0, 0, 1, 2, 5])))
    return specs


RANDOM = _random_window_specs(24)


@pytest.mark.parametrize("case", RANDOM, ids=[c["spec"].name for c in RANDOM])
def test_random_windowed_shapes_match_oracle(case):
    require_gpu()
    spec = case["spec"]
    announce(f"random window {spec}")
    w = W.make_workload(spec, device="cuda")
    out = run(w, num_splits=case["num_splits"])
    check_close(out.cpu().numpy(), oracle_full(w), spec.name)


@pytest.mark.parametrize("num_splits", [0, 1, 4])
def test_window_covering_every_position_is_bitwise_full_attention(num_splits):
    """W >= T visits the same tiles in the same order as no window, with nothing masked."""
    require_gpu()
    w = W.make_workload(W.preset("C4", batch=5, ctx=("uniform", 1, 900)), device="cuda")
    announce(f"window >= T vs full, num_splits={num_splits}")
    full = run(w, num_splits=num_splits)
    for window, sinks in ((900, 0), (901, 7), (1 << 20, 1 << 20)):
        win = run(w, num_splits=num_splits, window=window, num_sinks=sinks)
        assert torch.equal(full, win), (window, sinks)


@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_window_of_one_returns_the_last_value_row_exactly(num_splits):
    """softmax over one position is exactly 1, so the output is that position's V row."""
    require_gpu()
    spec = W.preset("C5", batch=3, ctx=(1000, 1, 17), window=1, num_sinks=0)
    w = W.make_workload(spec, device="cuda")
    announce(f"window 1, num_splits={num_splits}")
    out = run(w, num_splits=num_splits).cpu().numpy()
    v = W.oracle_view(w)
    vbits = v["v_cache"]
    g = spec.group
    for b, length in enumerate(v["ctx_lens"]):
        t = int(length) - 1
        blk, slot = int(v["block_table"][b, t // 16]), t % 16
        row = (vbits[blk, slot].astype(np.uint32) << 16).view(np.float32)  # [h_kv, d]
        want = np.repeat(row, g, axis=0)
        assert np.array_equal(out[b], want), b


def test_empty_sequences_with_a_window_give_zero_rows():
    require_gpu()
    spec = W.preset("C5", batch=3, ctx=(0, 500, 0), window=64, num_sinks=4)
    w = W.make_workload(spec, device="cuda")
    announce("window with empty sequences")
    for S in (0, 1, 2):
        out = run(w, num_splits=S)
        assert torch.count_nonzero(out[0]) == 0 and torch.count_nonzero(out[2]) == 0
        check_close(out.cpu().numpy(), oracle_full(w), f"empty rows S={S}")


def test_split_then_merge_equals_decode_with_a_window():
    require_gpu()
    from kv_cache_decode_split_amd import kv_attn as K
    spec = W.preset("C5", batch=2, ctx=(5000, 3001), window=1500, num_sinks=4)
    w = W.make_workload(spec, device="cuda")
    announce("window split+merge vs decode")
    a = torch.full(w.q.shape, float("nan"), device="cuda")
    b = torch.full(w.q.shape, float("nan"), device="cuda")
    call_a = K.decode_call_for(w, a, num_splits=4)
    call_b = K.decode_call_for(w, b, num_splits=4)
    assert call_a.plan()["num_splits"] == 4
    call_a.decode()
    call_b.split()
    call_b.merge()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


FULL = [
    # (preset, window, sinks, sampled sequences, sampled KV heads)
    ("C5", 4096, 4, [0, 3], [0, 5]),
    ("C4", 1024, 0, "extremes", [0, 7]),
    ("C3", 2000, 16, [0, 63], [3]),
]


@pytest.mark.parametrize("name,window,sinks,seqs,heads", FULL, ids=[f[0] for f in FULL])
def test_full_size_windowed_workloads_on_sampled_rows(name, window, sinks, seqs, heads):
    """Full-size workloads with a window, in the bench's launch configuration (auto plan)."""
    require_gpu()
    announce(f"full window {name} W={window} sinks={sinks}")
    w = W.make_workload(W.preset(name, window=window, num_sinks=sinks), device="cuda")
    try:
        out = run(w)
        assert torch.isfinite(out).all(), "non-finite output somewhere in the full batch"
        if seqs == "extremes":
            ctx = w.ctx_lens.cpu().numpy()
            order = np.argsort(ctx, kind="stable")
            seqs = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
        ref = oracle_rows(w, seqs, heads)
        check_close(select_rows(out, w, seqs, heads), ref, f"full window {name} seqs={seqs}")
    finally:
        del w
        torch.cuda.empty_cache()
