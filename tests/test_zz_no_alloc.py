"""kv_attn_decode_noalloc (the entry point that allocates nothing) against kv_attn_decode.

Two calls in a row through the C ABI on one device, the second with a smaller problem (so the
library's scratch still holds the first call's split states): each output must be bit-identical
to kv_attn_decode's on the same inputs (same plan, same kernels) and within the parity tolerance
of the fp64 oracle. A problem whose plan needs more than the fixed scratch is refused before
anything is launched.
"""

import ctypes

import pytest
import torch

from kv_cache_decode_split_amd import workloads as W
from tests.gpu_helpers import announce, check_close, oracle_full, require_gpu, run

pytestmark = pytest.mark.gpu


def _noalloc(K, w):
    out = torch.full(w.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    call = K.decode_call_for(w, out, allocate_workspace=False)
    assert call.workspace is None
    stream = torch.cuda.current_stream().cuda_stream
    st = K._lib.kv_attn_decode_noalloc(*call._ptrs, ctypes.byref(call.params), stream)
    assert st == K.KV_ATTN_OK, K.kv_attn_status_string(st)
    torch.cuda.synchronize()
    return out, call.plan()


def test_noalloc_matches_decode_on_two_calls_in_a_row():
    K = require_gpu()
    specs = [
        # paged, ragged, group 4 (rows mode), several splits per sequence
        W.preset("C4", batch=24, ctx=("uniform", 128, 30000)),
        # smaller: contiguous, group 1 (one-token MFMA kernel), a different split count
        W.preset("C2", batch=3, ctx=(5000, 1200, 77), capacity=5000),
    ]
    sizes = []
    for spec in specs:
        announce(f"noalloc {spec.name} batch={spec.batch}")
        w = W.make_workload(spec, device="cuda")
        want = run(w)
        got, plan = _noalloc(K, w)
        assert plan["num_splits"] > 1 and 0 < plan["workspace_bytes"] <= K.KV_ATTN_NOALLOC_SCRATCH_BYTES
        sizes.append(plan["workspace_bytes"])
        assert torch.equal(got, want), "noalloc output differs from kv_attn_decode's"
        check_close(got.cpu().numpy(), oracle_full(w), f"noalloc {spec.name}")
    assert sizes[1] < sizes[0]


def test_noalloc_refuses_a_plan_larger_than_its_scratch():
    K = require_gpu()
    p = K.make_params(batch=64, num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
                      max_ctx_len=1 << 20, num_blocks=1 << 26, max_blocks_per_seq=1 << 16,
                      k_strides=(8 * 16 * 128, 128, 16 * 128), v_strides=(8 * 16 * 128, 128, 16 * 128))
    assert K.kv_attn_workspace_size(p) > K.KV_ATTN_NOALLOC_SCRATCH_BYTES
    # Refused before any launch: the pointers are never dereferenced.
    st = K._lib.kv_attn_decode_noalloc(256, 256, 256, 256, 256, 256, ctypes.byref(p), None)
    assert st == K.KV_ATTN_ERR_SCRATCH
