"""GPU checks of the longest-first unit order: an order kernel lists the (sequence, split) pairs
whole splits first, then each sequence's last partial split by decreasing length, then a -1 for
each empty pair, and the split workgroups serve the pairs in that order. The planner picks it when the split
workgroups take several rounds of the device (C4 on a 256-CU MI355X); here it is forced
(KV_ATTN_UNIT_ORDER=1) on shapes the oracle checks in seconds, across the kernel variants, paged
and contiguous caches, ragged and empty sequences, several query tokens, sliding windows and wave
heads. Each pair's result does not depend on which workgroup serves it, so the output must also be
bit-identical to the split-by-split order.
"""

import numpy as np
import pytest
import torch

from kv_cache_decode_split_amd import workloads as W
from tests.gpu_helpers import announce, check_close, oracle_full, require_gpu
from tests.test_gpu_verify import oracle_verify

pytestmark = pytest.mark.gpu


def _decode(w, monkeypatch, order, num_splits):
    """Output of one decode with the unit order forced on or off, and the call (for its plan and
    workspace)."""
    K = require_gpu()
    monkeypatch.setenv("KV_ATTN_UNIT_ORDER", "1" if order else "0")
    out = torch.full(w.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    call = K.decode_call_for(w, out, num_splits=num_splits)
    assert call.plan()["unit_order"] == int(order)
    call.decode()
    torch.cuda.synchronize()
    return out, call


CASES = [
    ("C4", dict(batch=6, ctx=(0, 700, 1, 333, 2000, 1999))),                    # rows mode, g = 4
    ("C5", dict(batch=3, ctx=(3000, 17, 2048))),                                # rows mode, g = 8
    ("C2", dict(batch=4, ctx=(700, 1, 333, 512), num_q_heads=8, num_kv_heads=8, layers=1)),  # MFMA g = 1
    ("C1", dict(batch=3, ctx=(700, 1, 333), head_dim=128, num_q_heads=32, num_kv_heads=4,
                q_dtype="f32")),                                                # vector, g = 8
    ("C3", dict(batch=3, ctx=(1000, 17, 999), capacity=1000)),                  # contiguous
    ("C4", dict(batch=2, ctx=(900, 450), num_q_heads=24, num_kv_heads=12, head_dim=64)),  # g = 2
    ("C4", dict(batch=5, ctx=("uniform", 1, 700), num_queries=4)),              # several tokens
    ("C4", dict(batch=5, ctx=("uniform", 1, 700), window=100, num_sinks=16, extra_blocks=4)),
]


@pytest.mark.parametrize("name,over", CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(CASES)])
@pytest.mark.parametrize("num_splits", [3, 5])
def test_unit_order_matches_oracle_and_the_default_order(name, over, num_splits, monkeypatch):
    spec = W.preset(name, **over)
    announce(f"unit order {name} {over} num_splits={num_splits}")
    w = W.make_workload(spec, device="cuda")
    got, _ = _decode(w, monkeypatch, True, num_splits)
    ref = oracle_verify(w) if spec.num_queries > 1 else oracle_full(w)
    check_close(got.cpu().numpy(), ref, f"unit order {name} S={num_splits}")
    plain, _ = _decode(w, monkeypatch, False, num_splits)
    assert torch.equal(got, plain), "the order of the pairs changed a result"


def test_unit_order_with_wave_heads(monkeypatch):
    monkeypatch.setenv("KV_ATTN_WAVE_HEADS", "1")
    spec = W.preset("C5", batch=3, ctx=(3000, 2999, 5))
    w = W.make_workload(spec, device="cuda")
    got, call = _decode(w, monkeypatch, True, 4)
    assert call.plan()["wave_heads"] == 1
    check_close(got.cpu().numpy(), oracle_full(w), "unit order with wave heads")
    plain, _ = _decode(w, monkeypatch, False, 4)
    assert torch.equal(got, plain)


def _visited_tiles(ctx, max_ctx, window, sinks, nq):
    ctx = min(max(int(ctx), 0), max_ctx)
    if window is None:
        return -(-ctx // 16)
    sink_end = min(sinks, ctx)
    win_start = max(ctx - (nq - 1) - window, 0)
    n_first = -(-sink_end // 16)
    win_tile0 = max(win_start // 16, n_first)
    return n_first + max(-(-ctx // 16) - win_tile0, 0)


@pytest.mark.parametrize("over", [
    dict(batch=40, ctx=("uniform", 0, 5000)),
    dict(batch=33, ctx=("uniform", 1, 3000), window=500, num_sinks=4, extra_blocks=4),
])
def test_order_list_is_a_longest_first_permutation(over, monkeypatch):
    """The order kernel's list, read back from the workspace: every non-empty (sequence, split)
    pair once, whole splits first, then partial splits by non-increasing length class, then -1
    for each empty pair."""
    spec = W.preset("C4", **over)
    w = W.make_workload(spec, device="cuda")
    announce(f"order list {over}")
    _, call = _decode(w, monkeypatch, True, 6)
    plan = call.plan()
    B, S, st = spec.batch, plan["num_splits"], plan["split_len"] // 16
    raw = call.workspace[plan["order_offset"]:plan["order_offset"] + 8 * B * S]
    pairs = raw.cpu().numpy().view(np.int32).reshape(B * S, 2)
    order, listed = pairs[:, 0], pairs[:, 1]
    ctx = w.ctx_lens.cpu().numpy()
    size = {}
    for b in range(B):
        nt = _visited_tiles(ctx[b], w.max_ctx_len, spec.window, spec.num_sinks, spec.num_queries)
        for s in range(S):
            size[b * S + s] = min(max(nt - s * st, 0), st)
    busy = sorted(i for i, n in size.items() if n > 0)
    # every non-empty pair once, then one -1 per empty pair
    n_busy = len(busy)
    assert sorted(order[:n_busy].tolist()) == busy
    assert (order[n_busy:] == -1).all() and len(order) - n_busy == B * S - len(busy)
    # each pair carries its sequence's clamped length
    assert all(int(listed[i]) == min(max(int(ctx[int(order[i]) // S]), 0), w.max_ctx_len) for i in range(n_busy))
    sizes = [size[int(item)] for item in order[:n_busy]]
    # class of a pair: 0 whole, 1 + (255 - length class) partial
    cls = [0 if n == st else 1 + 255 - (n * 256 - 1) // st for n in sizes]
    assert cls == sorted(cls), "pairs out of the longest-first order"
    # whole splits come split by split
    whole_splits = [int(item) % S for item, c in zip(order[:n_busy], cls) if c == 0]
    assert whole_splits == sorted(whole_splits)
