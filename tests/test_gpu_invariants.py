"""GPU invariants the method fixes exactly, error paths that need a device, and the merge step.

* one position: the output is that position's value row, bit for bit (exp(0) = 1, 1·v/1 = v);
* paged through a random block table vs contiguous, and head-major vs token-major storage:
  bit-identical (block-table translation is pure addressing; same plan, same arithmetic order);
* run-to-run bitwise determinism (no atomics, fixed reduction orders);
* empty sequences give zero rows, NaN-poisoned slots past each sequence never leak;
* the split count and the score data path (matrix cores vs vector ALUs) change rounding only;
* the standalone merge agrees with the oracle's merge of running states.
"""

import math
import os

import numpy as np
import pytest
import torch

from kv_cache_decode_split_amd import workloads as W
from tests.gpu_helpers import announce, check_close, oracle_full, require_gpu, run

pytestmark = pytest.mark.gpu


def _value_rows_at(w, position=0):
    """Stored value rows (fp32) at logical ``position`` of every sequence: [B, h_kv, d]."""
    v = W.oracle_view(w)
    out = []
    for b in range(w.spec.batch):
        if v["block_table"] is None:
            blk, slot = b, position
        else:
            blk, slot = v["block_table"][b, position // v["block_size"]], position % v["block_size"]
        row = v["v_cache"][blk, slot]
        if row.dtype == np.uint16:
            row = (row.astype(np.uint32) << 16).view(np.float32)
        out.append(row.astype(np.float32))
    return np.stack(out)


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5"])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_single_position_is_bit_exact(name, num_splits):
    require_gpu()
    spec = W.preset(name, batch=3, ctx=(1, 1, 1)) if name != "C1" else W.preset(name, ctx=(1,))
    announce(f"T=1 {name} S={num_splits}")
    w = W.make_workload(spec, device="cuda")
    out = run(w, num_splits=num_splits).cpu().numpy()
    vrows = _value_rows_at(w)
    g = spec.group
    for b in range(spec.batch):
        for h in range(spec.num_q_heads):
            assert np.array_equal(out[b, h], vrows[b, h // g]), (b, h)


def _contiguous_copy(w):
    """The same logical cache as ``w`` (paged) laid out contiguously, in the same layout (so
    that the plan maps the work the same way)."""
    spec = w.spec
    B, hkv, d = spec.batch, spec.num_kv_heads, spec.head_dim
    T = w.max_ctx_len
    ks = torch.zeros((B, hkv, T, d), dtype=w.k_cache.dtype, device="cuda")
    vs = torch.zeros_like(ks)
    kv = w.k_cache.permute(0, 2, 1, 3) if spec.layout == "head_major" else w.k_cache
    vv = w.v_cache.permute(0, 2, 1, 3) if spec.layout == "head_major" else w.v_cache
    bt = w.block_table.cpu()
    bs = w.block_size
    for b in range(B):
        n = int(w.ctx_lens[b])
        t = torch.arange(n)
        blk = bt[b, t // bs].to(torch.int64).cuda()
        slot = (t % bs).cuda()
        ks[b, :, :n] = kv[blk, slot].permute(1, 0, 2)
        vs[b, :, :n] = vv[blk, slot].permute(1, 0, 2)
    if spec.layout == "token_major":
        ks, vs = ks.permute(0, 2, 1, 3).contiguous(), vs.permute(0, 2, 1, 3).contiguous()
    c = W.Workload(spec=W.preset(spec.name, paged=False, layout=spec.layout), q=w.q, k_cache=ks,
                   v_cache=vs, block_table=None, ctx_lens=w.ctx_lens, block_size=T, num_blocks=B)
    return c


@pytest.mark.parametrize("layout", ["head_major", "token_major"])
@pytest.mark.parametrize("num_splits", [0, 1, 4])
def test_paged_equals_contiguous_bitwise(layout, num_splits):
    require_gpu()
    spec = W.preset("C4", batch=6, ctx=("uniform", 1, 900), layout=layout, extra_blocks=5)
    announce(f"paged-vs-contiguous {layout} S={num_splits}")
    w = W.make_workload(spec, device="cuda")
    c = _contiguous_copy(w)
    a = run(w, num_splits=num_splits, max_ctx_len=w.max_ctx_len)
    b = run(c, num_splits=num_splits, max_ctx_len=w.max_ctx_len)
    assert torch.equal(a, b)


@pytest.mark.parametrize("wave_heads", [False, True])
def test_head_major_equals_token_major_bitwise(monkeypatch, wave_heads):
    """With the same mapping (one KV head per workgroup, or one per wave for both layouts) the
    layout changes addresses only."""
    K = require_gpu()
    monkeypatch.setenv("KV_ATTN_WAVE_HEADS", "1" if wave_heads else "0")
    ctx = (2000, 1777)
    hm = W.make_workload(W.preset("C5", batch=2, ctx=ctx, layout="head_major"), device="cuda")
    tm_k = hm.k_cache.permute(0, 2, 1, 3).contiguous()  # [N, bs, hkv, d]
    tm_v = hm.v_cache.permute(0, 2, 1, 3).contiguous()
    tm = W.Workload(spec=W.preset("C5", batch=2, ctx=ctx, layout="token_major"), q=hm.q,
                    k_cache=tm_k, v_cache=tm_v, block_table=hm.block_table, ctx_lens=hm.ctx_lens,
                    block_size=hm.block_size, num_blocks=hm.num_blocks)
    out = torch.empty(hm.q.shape, dtype=torch.float32, device="cuda")
    plans = [K.decode_call_for(x, out).plan() for x in (hm, tm)]
    assert plans[0] == plans[1] and plans[0]["wave_heads"] == int(wave_heads)
    assert torch.equal(run(hm), run(tm))


DETERMINISM = {
    "C1": W.preset("C1"),
    "C3": W.preset("C3", batch=4, ctx=(2048, 100, 1500, 9), capacity=2048),
    "C4": W.preset("C4", batch=4, ctx=("uniform", 1, 3000)),
}


@pytest.mark.parametrize("name", list(DETERMINISM))
def test_bitwise_determinism(name):
    require_gpu()
    w = W.make_workload(DETERMINISM[name], device="cuda")
    first = run(w)
    for _ in range(3):
        assert torch.equal(first, run(w))


def test_empty_sequences_give_zero_rows():
    require_gpu()
    for paged in (False, True):
        for S in (0, 1, 3):
            spec = W.preset("C4", batch=4, ctx=(0, 50, 0, 700), paged=paged,
                            capacity=None if paged else 700)
            w = W.make_workload(spec, device="cuda")
            out = run(w, num_splits=S)
            assert torch.all(out[0] == 0) and torch.all(out[2] == 0)
            check_close(out.cpu().numpy(), oracle_full(w), f"empty rows paged={paged} S={S}")


def test_all_sequences_empty():
    require_gpu()
    w = W.make_workload(W.preset("C3", batch=2, ctx=(0, 0), capacity=16), device="cuda")
    out = run(w, max_ctx_len=0)
    assert torch.all(out == 0)


def test_short_sequences_in_a_long_plan_leave_splits_empty():
    """max_ctx_len far above the real lengths: most split workgroups have nothing to do."""
    require_gpu()
    w = W.make_workload(W.preset("C4", batch=5, ctx=(1, 17, 33, 2, 16)), device="cuda")
    # Widen the table to 2048 columns (entries past each sequence point at the NaN block) so
    # that a 32768-position plan is valid for it.
    pad = torch.full((5, 2048 - w.block_table.shape[1]), int(w.block_table[0, -1]),
                     dtype=torch.int32, device="cuda")
    w.block_table = torch.cat([w.block_table, pad], dim=1).contiguous()
    out = run(w, max_ctx_len=32768, num_splits=0)
    check_close(out.cpu().numpy(), oracle_full(w), "short in long plan")


def test_context_lengths_beyond_max_are_clamped():
    require_gpu()
    w = W.make_workload(W.preset("C3", batch=2, ctx=(300, 300)), device="cuda")
    clamped = run(w, max_ctx_len=200)
    w2 = W.make_workload(W.preset("C3", batch=2, ctx=(300, 300)), device="cuda")
    w2.ctx_lens = torch.tensor([200, 200], dtype=torch.int32, device="cuda")
    assert torch.equal(clamped, run(w2, max_ctx_len=200))


@pytest.mark.parametrize("name", ["C2", "C3", "C5"])
def test_split_counts_agree(name):
    require_gpu()
    spec = W.preset(name, batch=2, ctx=(5000, 4001))
    w = W.make_workload(spec, device="cuda")
    ref = oracle_full(w)
    outs = {S: run(w, num_splits=S).cpu().numpy() for S in (1, 2, 7, 64, 313)}
    for S, o in outs.items():
        check_close(o, ref, f"{name} S={S}")
    assert np.max(np.abs(outs[1] - outs[313])) < 1e-4


def test_vector_and_matrix_core_paths_agree(monkeypatch):
    require_gpu()
    w = W.make_workload(W.preset("C5", batch=2, ctx=(3000, 1234)), device="cuda")
    mfma = run(w)
    monkeypatch.setenv("KV_ATTN_FORCE_VECTOR", "1")
    vec = run(w)
    monkeypatch.delenv("KV_ATTN_FORCE_VECTOR")
    ref = oracle_full(w)
    check_close(mfma.cpu().numpy(), ref, "mfma")
    check_close(vec.cpu().numpy(), ref, "vector")
    assert float((mfma - vec).abs().max()) < 1e-4


def test_non_default_stream():
    require_gpu()
    w = W.make_workload(W.preset("C3", batch=3, ctx=(900, 10, 400)), device="cuda")
    s = torch.cuda.Stream()
    out = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")
    from kv_cache_decode_split_amd import kv_attn as K
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        K.kv_attn_decode_workload(w, out)
    s.synchronize()
    check_close(out.cpu().numpy(), oracle_full(w), "side stream")


def test_workspace_too_small_is_rejected():
    K = require_gpu()
    w = W.make_workload(W.preset("C3", batch=2, ctx=(4000, 4000)), device="cuda")
    out = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(K.KvAttnError) as e:
        K.kv_attn_decode_workload(w, out, workspace=ws, num_splits=4)
    assert e.value.status == K.KV_ATTN_ERR_WORKSPACE


def test_debug_mode_validates_tables_before_launch(monkeypatch):
    """KV_ATTN_DEBUG=1 copies ctx_lens / block_table to the host and checks them first. The bad
    input used here (a length above max_ctx_len) is also clamped by the kernel, so even an
    unvalidated launch would stay in bounds."""
    K = require_gpu()
    w = W.make_workload(W.preset("C4", batch=3, ctx=(40, 50, 60)), device="cuda")
    out = torch.zeros(w.q.shape, dtype=torch.float32, device="cuda")
    monkeypatch.setenv("KV_ATTN_DEBUG", "1")
    K.kv_attn_decode_workload(w, out, max_ctx_len=60)  # valid tables pass
    check_close(out.cpu().numpy(), oracle_full(w), "debug mode")
    w.ctx_lens = torch.tensor([40, 61, 60], dtype=torch.int32, device="cuda")
    with pytest.raises(K.KvAttnError) as e:
        K.kv_attn_decode_workload(w, out, max_ctx_len=60)
    assert e.value.status == K.KV_ATTN_ERR_TABLE


# ---------------------------------------------------------------------------------------------
# the standalone merge (second pass) against the oracle's merge of running states


def _states(rng, rows, S, d, empty_frac=0.2):
    """Random split states built by the oracle from random blocks (natural-log maxima)."""
    from oracle import block_state
    states = []
    for r in range(rows):
        row = []
        for s in range(S):
            if rng.random() < empty_frac:
                row.append((-math.inf, 0.0, np.zeros(d)))
                continue
            n = int(rng.integers(1, 40))
            scores = rng.standard_normal(n) * 4 + rng.standard_normal() * 6
            values = rng.standard_normal((n, d))
            row.append(block_state(scores, values))
        states.append(row)
    return states


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("with_counts", [False, True])
def test_merge_matches_oracle(d, with_counts):
    K = require_gpu()
    from oracle import finalize_state, merge_many
    rng = np.random.default_rng(42 + d)
    rows, S = 37, 9
    states = _states(rng, rows, S, d)
    counts = rng.integers(0, S + 1, rows) if with_counts else np.full(rows, S)
    if with_counts:
        counts[0] = 0
    o = np.zeros((rows, S, d), dtype=np.float32)
    ml = np.zeros((rows, S, 2), dtype=np.float32)
    log2e = 1.0 / math.log(2.0)
    for r in range(rows):
        for s in range(S):
            m, l, acc = states[r][s]
            o[r, s] = acc
            ml[r, s] = (m * log2e if m != -math.inf else -math.inf, l)
    out = torch.full((rows, d), float("nan"), device="cuda")
    K.kv_attn_merge(torch.from_numpy(o).cuda(), torch.from_numpy(ml).cuda(),
                    torch.from_numpy(counts.astype(np.int32)).cuda() if with_counts else None, out)
    torch.cuda.synchronize()
    # Expected: the oracle merges the float32-rounded states it handed over.
    ref = np.zeros((rows, d))
    for r in range(rows):
        rounded = []
        for s in range(int(counts[r])):
            m, l, acc = states[r][s]
            rounded.append((float(np.float32(m)) if m != -math.inf else -math.inf,
                            float(np.float32(l)), o[r, s].astype(np.float64)))
        ref[r] = finalize_state(merge_many(rounded, d))
    got = out.cpu().numpy()
    if with_counts:
        assert np.all(got[0] == 0)
    np.testing.assert_allclose(got, ref, rtol=2e-5, atol=2e-5)
