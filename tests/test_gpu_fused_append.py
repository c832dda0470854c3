"""GPU checks of the fused append: in the bf16 matrix-core variants kv_attn_append_decode does not
launch the append kernel; the split workgroup whose tile holds the new tokens takes their K/V rows
from k_new / v_new and writes them into the cache. Two copies of each seeded workload run the two
ways (kv_attn_append then kv_attn_decode, and kv_attn_append_decode): the caches must be
bit-identical afterwards (every byte, the poisoned slots included), and the outputs equal up to
the rounding of a different visiting order (the split holding the new rows visits its tiles in
order, where the plain decode rotates them); both are also checked against the fp64 oracle on
the oracle-appended cache. The shapes cover one and
several query tokens, head dims 64 and 128, paged and contiguous caches, both layouts, windows,
explicit split counts that put the new rows at a split boundary, wave heads, the longest-first
unit order, empty and one-token sequences, and an fp32 cache (the separate append kernel).
"""

import numpy as np
import pytest
import torch

from kv_cache_decode_split_amd import workloads as W
from tests.gpu_helpers import announce, check_close, require_gpu
from tests.test_gpu_verify import oracle_verify
from tests.gpu_helpers import oracle_full

pytestmark = pytest.mark.gpu


def _new_rows(w, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    nq = max(w.spec.num_queries, 1)
    shape = ((w.spec.batch, w.spec.num_kv_heads, w.spec.head_dim) if nq == 1 else
             (w.spec.batch, nq, w.spec.num_kv_heads, w.spec.head_dim))
    k = torch.randn(shape, generator=g).to(w.k_cache.dtype).to(w.k_cache.device)
    v = torch.randn(shape, generator=g).to(w.v_cache.dtype).to(w.v_cache.device)
    return k, v


def _poison_new_slots(w):
    """NaN in every slot the new tokens go to, so a slot read before it is written shows."""
    nq = max(w.spec.num_queries, 1)
    ctx = w.ctx_lens.cpu().tolist()
    bt = None if w.block_table is None else w.block_table.cpu()
    for b, t in enumerate(ctx):
        if t < nq:
            continue
        for p in range(t - nq, t):
            blk, slot = (b, p) if bt is None else (int(bt[b, p // w.block_size]), p % w.block_size)
            if w.spec.layout == "token_major":
                w.k_cache[blk, slot].fill_(float("nan"))
                w.v_cache[blk, slot].fill_(float("nan"))
            else:
                w.k_cache[blk, :, slot].fill_(float("nan"))
                w.v_cache[blk, :, slot].fill_(float("nan"))


def _raw(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


CASES = [
    ("C4", dict(batch=6, ctx=("uniform", 1, 900)), {}),                            # rows mode
    ("C2", dict(batch=3, ctx=(700, 0, 1), layers=1), {}),                          # variant 1, g = 1
    ("C2", dict(batch=2, ctx=(513, 40), num_q_heads=16, num_kv_heads=8, layers=1), {}),  # g = 2
    ("C4", dict(batch=3, ctx=(900, 17, 450), num_q_heads=24, num_kv_heads=12, head_dim=64), {}),
    ("C3", dict(batch=3, ctx=(1000, 17, 999), capacity=1000), {}),                 # contiguous
    ("C4", dict(batch=5, ctx=("uniform", 1, 300), layout="token_major", extra_blocks=3), {}),
    ("C5", dict(batch=2, ctx=(4098, 4097)), dict(num_splits=3)),                   # split boundary
    # 4 tokens; S = 2 of 65 tiles: sequence 1's new rows 1038..1041 straddle the split boundary
    ("C4", dict(batch=4, ctx=(2080, 1042, 3, 700), num_queries=4), dict(num_splits=2)),
    ("C4", dict(batch=3, ctx=(2050, 2, 700), num_queries=2, head_dim=64), {}),
    ("C4", dict(batch=5, ctx=("uniform", 1, 700), window=100, num_sinks=16, extra_blocks=4), {}),
    ("C1", dict(batch=2, ctx=(300, 5), capacity=320), {}),                          # fp32: append kernel
]


def _run(name, over, kw, monkeypatch, env=None):
    K = require_gpu()
    for k, v in (env or {}).items():
        monkeypatch.setenv(k, v)
    spec = W.preset(name, **over)
    nq = max(spec.num_queries, 1)
    outs, caches = [], []
    for fused in (False, True):
        w = W.make_workload(spec, device="cuda")
        _poison_new_slots(w)
        k_new, v_new = _new_rows(w, 29)
        out = torch.full(w.q.shape, float("nan"), dtype=torch.float32, device="cuda")
        call = K.decode_call_for(w, out, **kw)
        if fused:
            call.append_decode(k_new, v_new)
        else:
            ks, vs = w.kv_strides()
            pos = (w.ctx_lens - nq).to(torch.int32)
            pos = torch.where(w.ctx_lens >= nq, pos, torch.full_like(pos, -1))
            K.kv_attn_append(k_new, v_new, w.k_cache, w.v_cache, w.block_table, pos,
                             num_kv_heads=spec.num_kv_heads, k_strides=ks, v_strides=vs,
                             block_size=w.block_size, num_blocks=w.num_blocks)
            call.decode()
        torch.cuda.synchronize()
        outs.append(out)
        caches.append((w.k_cache.clone(), w.v_cache.clone()))
        last = w
    assert torch.equal(_raw(caches[0][0]), _raw(caches[1][0])), "K caches differ"
    assert torch.equal(_raw(caches[0][1]), _raw(caches[1][1])), "V caches differ"
    diff = (outs[0] - outs[1]).abs().max().item()
    assert diff <= 1e-5 * max(outs[0].abs().max().item(), 1e-30), f"outputs differ by {diff}"
    ref = oracle_verify(last) if nq > 1 else oracle_full(last)
    check_close(outs[0].cpu().numpy(), ref, f"append then decode {name} {over}")
    check_close(outs[1].cpu().numpy(), ref, f"fused append {name} {over}")


@pytest.mark.parametrize("name,over,kw", CASES, ids=[f"{n}-{i}" for i, (n, _, _) in enumerate(CASES)])
def test_fused_append_equals_append_then_decode(name, over, kw, monkeypatch):
    announce(f"fused append {name} {over} {kw}")
    _run(name, over, kw, monkeypatch)


def test_fused_append_with_wave_heads(monkeypatch):
    announce("fused append, wave heads")
    _run("C5", dict(batch=2, ctx=(3000, 2999)), {}, monkeypatch, env={"KV_ATTN_WAVE_HEADS": "1"})


def test_fused_append_with_unit_order(monkeypatch):
    announce("fused append, unit order")
    _run("C4", dict(batch=6, ctx=(0, 700, 1, 333, 2000, 1999)), dict(num_splits=5), monkeypatch,
         env={"KV_ATTN_UNIT_ORDER": "1"})
