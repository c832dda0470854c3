"""GPU parity of the wave-heads mapping: each wave of a split workgroup serves its own KV head and
streams a whole split. The planner picks it for long sequences with few (sequence, KV head) units;
here it is forced (KV_ATTN_WAVE_HEADS=1) on shapes the oracle checks in seconds, across every
kernel variant, both cache layouts, paged and contiguous caches, ragged and empty sequences,
several query tokens, sliding windows and score export, each with the automatic, one and three
splits.
"""

import pytest
import torch

from kv_cache_decode_split_amd import workloads as W
from tests.gpu_helpers import announce, check_close, oracle_full, require_gpu, run
from tests.test_gpu_scores import _check_output, _oracle_scores, _run_scores
from tests.test_gpu_verify import oracle_verify

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _force_wave_heads(monkeypatch):
    monkeypatch.setenv("KV_ATTN_WAVE_HEADS", "1")


def _plan(w, **kw):
    K = require_gpu()
    out = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")
    return K.decode_call_for(w, out, **kw).plan()


DECODE = [
    ("C5", dict(batch=2, ctx=(3000, 2999))),                                   # rows mode, g = 8
    ("C5", dict(batch=2, ctx=(3000, 17), layout="token_major")),
    ("C2", dict(batch=3, ctx=(700, 1, 333), num_q_heads=8, num_kv_heads=8, layers=1)),  # g = 1
    ("C1", dict(batch=3, ctx=(700, 1, 333), head_dim=128, num_q_heads=32, num_kv_heads=4,
                q_dtype="f32", layout="token_major")),                         # vector, g = 8
    ("C4", dict(batch=4, ctx=(0, 700, 1, 333))),                               # empty sequence
    ("C3", dict(batch=3, ctx=(1000, 17, 999), capacity=1000, layout="token_major")),  # contiguous
    ("C4", dict(batch=2, ctx=(900, 450), num_q_heads=24, num_kv_heads=12, head_dim=64)),  # g = 2
    ("C4", dict(batch=3, ctx=(600, 5, 256), num_q_heads=16, num_kv_heads=4, kv_dtype="f32",
                q_dtype="bf16", layout="token_major")),                        # mixed dtypes
]


@pytest.mark.parametrize("name,over", DECODE, ids=[f"{n}-{i}" for i, (n, _) in enumerate(DECODE)])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_decode_matches_oracle(name, over, num_splits):
    spec = W.preset(name, **over)
    announce(f"wave heads decode {name} {over} num_splits={num_splits}")
    w = W.make_workload(spec, device="cuda")
    assert _plan(w, num_splits=num_splits)["wave_heads"] == 1
    out = run(w, num_splits=num_splits)
    check_close(out.cpu().numpy(), oracle_full(w), f"{name} S={num_splits}")


VERIFY = [
    ("C5", dict(batch=2, ctx=(3000, 1777)), 2),                                # 16 rows, one block
    ("C5", dict(batch=2, ctx=(3000, 2), layout="token_major"), 4),             # 32 rows, two blocks
    ("C3", dict(batch=3, ctx=(1000, 77, 4), capacity=1010), 4),
    ("C4", dict(batch=5, ctx=("uniform", 1, 700), layout="token_major"), 8),
]


@pytest.mark.parametrize("name,over,gamma", VERIFY, ids=[f"{n}-g{g}-{i}" for i, (n, _, g) in enumerate(VERIFY)])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_verification_matches_oracle(name, over, gamma, num_splits):
    spec = W.preset(name, num_queries=gamma, **over)
    announce(f"wave heads verify {name} {over} gamma={gamma} num_splits={num_splits}")
    w = W.make_workload(spec, device="cuda")
    assert _plan(w, num_splits=num_splits)["wave_heads"] == 1
    out = run(w, num_splits=num_splits)
    check_close(out.cpu().numpy(), oracle_verify(w), f"{name} gamma={gamma} S={num_splits}")


WINDOWED = [
    ("C5", dict(batch=2, ctx=(3000, 2999)), 1, 1000, 4),
    ("C4", dict(batch=5, ctx=("uniform", 1, 700), layout="token_major", extra_blocks=4), 1, 100, 16),
    ("C5", dict(batch=2, ctx=(1500, 33), layout="token_major"), 4, 17, 5),   # edges inside tiles
]


@pytest.mark.parametrize("name,over,gamma,window,sinks", WINDOWED,
                         ids=[f"{n}-W{wd}-{i}" for i, (n, _, _, wd, _) in enumerate(WINDOWED)])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_windowed_matches_oracle(name, over, gamma, window, sinks, num_splits):
    spec = W.preset(name, num_queries=gamma, window=window, num_sinks=sinks, **over)
    announce(f"wave heads window {name} {over} gamma={gamma} W={window} n={sinks} S={num_splits}")
    w = W.make_workload(spec, device="cuda")
    assert _plan(w, num_splits=num_splits)["wave_heads"] == 1
    out = run(w, num_splits=num_splits)
    ref = oracle_verify(w) if gamma > 1 else oracle_full(w)
    check_close(out.cpu().numpy(), ref, f"{name} W={window} S={num_splits}")


SCORES = [
    ("C5", dict(batch=2, ctx=(3000, 1777))),
    ("C4", dict(batch=5, ctx=("uniform", 1, 700), layout="token_major")),
    ("C2", dict(batch=3, ctx=(700, 0, 333), num_q_heads=8, num_kv_heads=8, layers=1)),
]


@pytest.mark.parametrize("name,over", SCORES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(SCORES)])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_score_export_matches_oracle(name, over, num_splits):
    spec = W.preset(name, **over)
    announce(f"wave heads scores {name} {over} num_splits={num_splits}")
    w = W.make_workload(spec, device="cuda")
    assert _plan(w, num_splits=num_splits)["wave_heads"] == 1
    out, scores = _run_scores(w, num_splits=num_splits)
    check_close(scores.cpu().numpy(), _oracle_scores(w), f"scores {name} S={num_splits}")
    _check_output(out, w, num_splits, f"scores {name} S={num_splits}")


@pytest.mark.parametrize("layout", ["head_major", "token_major"])
def test_split_then_merge_equals_decode(layout):
    K = require_gpu()
    spec = W.preset("C5", batch=2, ctx=(5000, 3001), layout=layout)
    w = W.make_workload(spec, device="cuda")
    announce(f"wave heads split+merge vs decode {layout}")
    a = torch.full(w.q.shape, float("nan"), device="cuda")
    b = torch.full(w.q.shape, float("nan"), device="cuda")
    call_a = K.decode_call_for(w, a, num_splits=4)
    call_b = K.decode_call_for(w, b, num_splits=4)
    assert call_a.plan()["wave_heads"] == 1 and call_a.plan()["num_splits"] == 4
    call_a.decode()
    call_b.split()
    call_b.merge()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    check_close(a.cpu().numpy(), oracle_full(w), f"split+merge {layout}")
