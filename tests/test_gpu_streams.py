"""Launches on a stream other than the current one, through the one-shot wrappers.

The wrappers allocate their workspace (and the eviction mask, when none is given) from torch's
caching allocator on the current stream and drop it as soon as the kernels are enqueued. With
``stream=`` naming another stream, the allocator must not hand that memory to new work on the
current stream while the kernels still use it: right after each call the tests allocate
same-sized buffers on the current stream and fill them with garbage, then check the results
against the oracle.
"""

import numpy as np
import pytest
import torch

from kv_cache_decode_split_amd import workloads as W
from tests.gpu_helpers import announce, check_close, oracle_full, require_gpu

pytestmark = pytest.mark.gpu


def _scribble(nbytes: int, rounds: int = 4):
    """Allocate and fill buffers of ``nbytes`` on the current stream (what a caller might do next)."""
    held = []
    for _ in range(rounds):
        t = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        t.fill_(0xFF)  # NaN patterns in fp32
        held.append(t)
    return held


def test_decode_on_a_side_stream_keeps_its_workspace():
    K = require_gpu()
    announce("decode on a side stream, one-shot wrapper")
    spec = W.preset("C5", batch=2, ctx=(60000, 41000))  # several splits: the workspace is used
    w = W.make_workload(spec, device="cuda")
    out = torch.full(w.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    call = K.decode_call_for(w, out)
    plan = call.plan()
    assert plan["num_splits"] > 1
    nbytes = plan["workspace_bytes"]
    del call
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    held = []
    for _ in range(3):
        K.kv_attn_decode_workload(w, out, stream=side)
        held += _scribble(nbytes)
    torch.cuda.synchronize()
    check_close(out.cpu().numpy(), oracle_full(w), "side-stream decode")


def test_eviction_on_a_side_stream_keeps_its_workspace():
    require_gpu()
    from kv_cache_decode_split_amd import kv_evict as E
    from oracle import evict_select

    announce("eviction on a side stream, one-shot wrapper")
    L, H, N = 4, 8, 8192
    scores = W.make_scores(L, H, N, "lognormal", seed=77, device="cuda")
    budget = L * H * N // 5
    need = E.kv_evict_workspace_size(E.make_evict_params(L, H, N, budget))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    held = []
    keeps = []
    for _ in range(3):
        keeps.append(E.kv_evict_select(scores, budget, stream=side))
        held += _scribble(need)
    torch.cuda.synchronize()
    want = evict_select(scores.cpu().numpy(), budget)
    for keep in keeps:
        assert np.array_equal(keep.cpu().numpy().astype(bool), np.asarray(want, dtype=bool))
