"""GPU tests of the KV append (the step before attention) and of append + decode in one call.

Expected caches come from ``oracle.append_kv`` applied to host copies of the caches taken before
the GPU call; expected attention outputs from the fp64 oracle on that oracle-appended cache.
Appends are bit-exact copies, compared as raw bits (NaN poison included).
"""

import numpy as np
import pytest
import torch

from kv_cache_decode_split_amd import workloads as W
from tests.gpu_helpers import announce, check_close, require_gpu

pytestmark = pytest.mark.gpu


def _bits(a):
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


def _new_rows(w, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    shape = (w.spec.batch, w.spec.num_kv_heads, w.spec.head_dim)
    k = torch.randn(shape, generator=g).to(w.k_cache.dtype).to(w.k_cache.device)
    v = torch.randn(shape, generator=g).to(w.v_cache.dtype).to(w.v_cache.device)
    return k, v


def _np_rows(t):
    t = t.cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


CASES = [
    W.preset("C4", batch=5, ctx=("uniform", 1, 200)),
    W.preset("C4", batch=4, ctx=("uniform", 1, 90), layout="token_major", block_size=32),
    W.preset("C3", batch=3, ctx=(40, 17, 63), capacity=64),
    W.preset("C1", batch=2, ctx=(30, 5), capacity=40, layout="token_major"),
]


@pytest.mark.parametrize("spec", CASES, ids=[f"{s.name}-{s.layout}-{'paged' if s.paged else 'contig'}" for s in CASES])
def test_append_matches_oracle_bitwise(spec):
    K = require_gpu()
    from oracle import append_kv
    announce(f"append {spec}")
    w = W.make_workload(spec, device="cuda")
    before = W.oracle_view(w)
    k_new, v_new = _new_rows(w, 7)
    ctx = w.ctx_lens.cpu().numpy()
    pos = np.array([int(t) for t in ctx], dtype=np.int32)  # the slot just past each sequence...
    pos[0] = -1                                             # ...except an idle sequence
    if w.block_table is not None:  # only positions whose block is in the table are valid
        cap = w.block_table.shape[1] * w.block_size
        pos = np.where(pos >= cap, pos - 1, pos)
    else:
        pos = np.minimum(pos, w.block_size - 1)
    positions = torch.from_numpy(pos).cuda()
    ks, vs = w.kv_strides()
    K.kv_attn_append(k_new, v_new, w.k_cache, w.v_cache, w.block_table, positions,
                     num_kv_heads=spec.num_kv_heads, k_strides=ks, v_strides=vs,
                     block_size=w.block_size, num_blocks=w.num_blocks)
    torch.cuda.synchronize()
    after = W.oracle_view(w)
    table = before["block_table"]
    kw = dict(block_size=w.block_size) if table is not None else dict(capacity=w.block_size)
    want_k = append_kv(before["k_cache"], _np_rows(k_new), pos, table, **kw)
    want_v = append_kv(before["v_cache"], _np_rows(v_new), pos, table, **kw)
    assert np.array_equal(_bits(np.ascontiguousarray(after["k_cache"])), _bits(want_k))
    assert np.array_equal(_bits(np.ascontiguousarray(after["v_cache"])), _bits(want_v))


def test_append_skips_out_of_range_positions():
    K = require_gpu()
    w = W.make_workload(W.preset("C3", batch=2, ctx=(10, 10), capacity=12), device="cuda")
    k0, v0 = w.k_cache.clone(), w.v_cache.clone()
    k_new, v_new = _new_rows(w, 3)
    ks, vs = w.kv_strides()
    K.kv_attn_append(k_new, v_new, w.k_cache, w.v_cache, None,
                     torch.tensor([12, -5], dtype=torch.int32, device="cuda"),
                     num_kv_heads=8, k_strides=ks, v_strides=vs, block_size=12, num_blocks=2)
    torch.cuda.synchronize()
    assert torch.equal(k0.view(torch.int16), w.k_cache.view(torch.int16))
    assert torch.equal(v0.view(torch.int16), w.v_cache.view(torch.int16))


def _poison_current_token(w):
    """NaN at position ctx_lens[b]-1 of every sequence: only a real append makes it readable."""
    bt = None if w.block_table is None else w.block_table.cpu()
    kv = w.k_cache.permute(0, 2, 1, 3) if w.spec.layout == "head_major" else w.k_cache
    vv = w.v_cache.permute(0, 2, 1, 3) if w.spec.layout == "head_major" else w.v_cache
    for b, t in enumerate(w.ctx_lens.cpu().tolist()):
        if t <= 0:
            continue
        p = t - 1
        blk, slot = (b, p) if bt is None else (int(bt[b, p // w.block_size]), p % w.block_size)
        kv[blk, slot].fill_(float("nan"))
        vv[blk, slot].fill_(float("nan"))


APPEND_DECODE = [
    ("C4", dict(batch=6, ctx=("uniform", 1, 900)), None),
    ("C5", dict(batch=2, ctx=(3000, 1777)), None),
    ("C2", dict(batch=2, ctx=(700, 0)), None),
    ("C4", None, [0, 64, 127]),   # full size, sampled sequences
]


@pytest.mark.parametrize("name,over,sample", APPEND_DECODE, ids=["C4-small", "C5-small", "C2-empty", "C4-full"])
def test_append_decode_matches_oracle(name, over, sample):
    K = require_gpu()
    from oracle import append_kv, decode_attention
    spec = W.PRESETS[name] if over is None else W.preset(name, **over)
    announce(f"append_decode {name} {over}")
    w = W.make_workload(spec, device="cuda")
    _poison_current_token(w)
    seqs = list(range(spec.batch)) if sample is None else sample
    before = W.oracle_sample(w, seqs)  # host copy before the GPU writes anything
    k_new, v_new = _new_rows(w, 11)
    out = torch.full(w.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    call = K.decode_call_for(w, out)
    call.append_decode(k_new, v_new)
    torch.cuda.synchronize()
    pos = before["ctx_lens"] - 1
    table = before["block_table"]
    kw = dict(block_size=before["block_size"]) if table is not None else dict(capacity=before["block_size"])
    kc = append_kv(before["k_cache"], _np_rows(k_new)[seqs], pos, table, **kw)
    vc = append_kv(before["v_cache"], _np_rows(v_new)[seqs], pos, table, **kw)
    ref = decode_attention(before["q"], kc, vc, before["ctx_lens"], table,
                           block_size=before["block_size"] if table is not None else None)
    check_close(out[seqs].cpu().numpy(), ref, f"append_decode {name}")
    if sample is not None:
        assert torch.isfinite(out).all()
