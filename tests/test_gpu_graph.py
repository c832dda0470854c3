"""The library under HIP graph capture (torch.cuda.CUDAGraph): captured launches replay the same
kernels with the same arguments, so every replay must equal the eager result bit for bit, with
the program's own eager work and synchronisations between replays, and must read inputs live.
The path records no memset or copy nodes (its only device writes are its own kernels)."""

import pytest
import torch

from kv_cache_decode_split_amd import workloads as W
from tests.gpu_helpers import announce, require_gpu

pytestmark = pytest.mark.gpu

CASES = {
    "C3-unsplit": (W.preset("C3", batch=2, ctx=(1000, 333)), 1),
    "C5-split": (W.preset("C5", batch=2, ctx=(3000, 1777)), 0),
    "C4-ragged": (W.preset("C4", batch=5, ctx=("uniform", 1, 2000)), 0),
}


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up launch off the default stream, as capture expects
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name", list(CASES))
def test_decode_graph_replays_equal_eager(name):
    K = require_gpu()
    spec, S = CASES[name]
    announce(f"graph decode {name}")
    w = W.make_workload(spec, device="cuda")
    out = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")
    call = K.decode_call_for(w, out, num_splits=S)
    call.decode()
    torch.cuda.synchronize()
    eager = out.clone()
    g = _capture(call.decode)
    scratch = torch.zeros(1 << 20, device="cuda")
    for i in range(4):
        out.fill_(float("nan"))
        scratch.add_(float(i))            # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager result"
    # inputs are read live: flip q, replay, and compare with a fresh eager launch
    w.q.mul_(-1)
    g.replay()
    torch.cuda.synchronize()
    replayed = out.clone()
    call.decode()
    torch.cuda.synchronize()
    assert torch.equal(replayed, out)
    assert not torch.equal(replayed, eager)


def test_append_decode_graph_replays_equal_eager():
    K = require_gpu()
    w = W.make_workload(W.preset("C4", batch=4, ctx=("uniform", 2, 700)), device="cuda")
    out = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(5)
    shape = (4, 8, 128)
    kn = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
    vn = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
    call = K.decode_call_for(w, out)
    call.append_decode(kn, vn)
    torch.cuda.synchronize()
    eager = out.clone()
    g = _capture(lambda: call.append_decode(kn, vn))
    for i in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"


def _check_replays(g, outputs, eager, label, reps=4):
    scratch = torch.zeros(1 << 20, device="cuda")
    for i in range(reps):
        for o in outputs:
            o.fill_(float("nan")) if o.dtype.is_floating_point else o.fill_(0xAB)
        scratch.add_(float(i))            # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outputs, eager):
            assert torch.equal(o, e), f"{label}: replay {i} differs from the eager result"


def test_verification_decode_graph_replays_equal_eager():
    K = require_gpu()
    w = W.make_workload(W.preset("C5", batch=2, ctx=(3000, 1777), num_queries=4), device="cuda")
    out = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")
    call = K.decode_call_for(w, out)
    call.decode()
    torch.cuda.synchronize()
    eager = out.clone()
    _check_replays(_capture(call.decode), [out], [eager], "verify")


def test_score_export_graph_replays_equal_eager():
    K = require_gpu()
    w = W.make_workload(W.preset("C4", batch=4, ctx=("uniform", 1, 2000)), device="cuda")
    out = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")
    scores = torch.empty((4, w.spec.num_kv_heads, w.max_ctx_len), dtype=torch.float32, device="cuda")
    call = K.decode_call_for(w, out, with_scores=True)
    call.decode_scores(scores)
    torch.cuda.synchronize()
    eager = [out.clone(), scores.clone()]
    _check_replays(_capture(lambda: call.decode_scores(scores)), [out, scores], eager, "scores")


def test_eviction_selection_graph_replays_equal_eager():
    require_gpu()
    from kv_cache_decode_split_amd import kv_evict as E
    s = W.make_scores(8, 8, 4096, "lognormal", seed=3, device="cuda")
    budget = 8 * 8 * 4096 // 7
    keep = torch.empty((8, 8, 4096), dtype=torch.uint8, device="cuda")
    counts = torch.empty((8, 8), dtype=torch.int32, device="cuda")
    p = E.make_evict_params(8, 8, 4096, budget)
    ws = torch.empty(E.kv_evict_workspace_size(p), dtype=torch.uint8, device="cuda")

    def call():
        E.kv_evict_select(s, budget, keep=keep, kept_per_row=counts, workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = [keep.clone(), counts.clone()]
    g = _capture(call)
    _check_replays(g, [keep, counts], eager, "evict")
    # inputs are read live: different scores through the same graph
    s.mul_(-1.0)
    g.replay()
    torch.cuda.synchronize()
    replayed = keep.clone()
    call()
    torch.cuda.synchronize()
    assert torch.equal(replayed, keep) and not torch.equal(replayed, eager[0])
