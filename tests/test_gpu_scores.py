"""GPU parity of decode with score export (kv_attn_decode_scores) against the fp64 oracle.

The exported weights are compared with ``oracle.position_scores`` at the parity tolerance; the
attention output of the same call must equal plain kv_attn_decode bit for bit where both run
the same kernel (the export only adds stores; plain decode of bf16 groups of 4 or more runs the
rows-mode kernel instead, and the output is then compared with the oracle); accumulation adds
exactly and leaves unattended entries alone; and a decode ->
scores -> eviction pipeline over several layers selects exactly what the oracle selection picks
from the same scores.
"""

import numpy as np
import pytest
import torch

from kv_cache_decode_split_amd import workloads as W
from tests.gpu_helpers import announce, check_close, oracle_full, require_gpu, run

pytestmark = pytest.mark.gpu


def _oracle_scores(w, seqs=None, kv_heads=None):
    from oracle import position_scores
    v = W.oracle_view(w) if seqs is None else W.oracle_sample(w, seqs, kv_heads)
    kw = {} if w.spec.window is None else dict(window=w.spec.window, num_sinks=w.spec.num_sinks)
    paged = v["block_table"] is not None
    return position_scores(v["q"], v["k_cache"], v["ctx_lens"], v["block_table"],
                           block_size=v["block_size"] if paged else None,
                           max_len=w.max_ctx_len, **kw)


def _check_output(out, w, num_splits, label):
    """The output of a score-export call: the plain decode's bits (score export runs the same
    kernel variant and plan, with the score stores added), and within the parity tolerance of
    the oracle."""
    assert torch.equal(out, run(w, num_splits=num_splits)), "score export changed the output"
    check_close(out.cpu().numpy(), oracle_full(w), f"{label} output")


def _run_scores(w, accumulate=False, fill=float("nan"), **kwargs):
    K = require_gpu()
    out = torch.full(w.q.shape, float("nan"), dtype=torch.float32, device=w.q.device)
    scores = torch.full((w.spec.batch, w.spec.num_kv_heads, w.max_ctx_len), fill,
                        dtype=torch.float32, device=w.q.device)
    call = K.decode_call_for(w, out, with_scores=True, **kwargs)
    call.decode_scores(scores, accumulate=accumulate)
    torch.cuda.synchronize()
    return out, scores


SMALL = [
    ("C1", dict()),                                                        # fp32 vector path
    ("C2", dict(batch=2, ctx=(700, 333), layers=1)),                       # g = 1
    ("C3", dict(batch=3, ctx=(1000, 77, 1), capacity=1010)),               # g = 4, contiguous
    ("C4", dict(batch=6, ctx=("uniform", 1, 900), layout="token_major")),  # ragged, paged
    ("C4", dict(batch=3, ctx=(0, 300, 17))),                               # an empty sequence
    ("C5", dict(batch=2, ctx=(3000, 1777))),                               # g = 8, sinks
    ("C5", dict(batch=2, ctx=(900, 333), num_q_heads=16, num_kv_heads=1, head_dim=64)),  # g = 16
    ("C1", dict(batch=2, ctx=(256, 100), head_dim=128, num_q_heads=16, num_kv_heads=2)),
    ("C1", dict(batch=2, ctx=(500, 90), head_dim=128, num_q_heads=32, num_kv_heads=2)),  # g = 16, halves
]


@pytest.mark.parametrize("name,over", SMALL, ids=[f"{n}-{i}" for i, (n, _) in enumerate(SMALL)])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_exported_weights_match_oracle(name, over, num_splits):
    K = require_gpu()
    spec = W.preset(name, **over)
    announce(f"scores {name} {over} num_splits={num_splits}")
    w = W.make_workload(spec, device="cuda")
    out, scores = _run_scores(w, num_splits=num_splits)
    ref = _oracle_scores(w)
    check_close(scores.cpu().numpy(), ref, f"scores {name} S={num_splits}")
    _check_output(out, w, num_splits, f"scores {name} S={num_splits}")
    lens = w.ctx_lens.cpu().numpy()
    sums = scores.double().sum(-1).cpu().numpy()
    for b, length in enumerate(lens):
        np.testing.assert_allclose(sums[b], spec.group if length > 0 else 0.0, rtol=1e-4, atol=1e-6)


@pytest.mark.parametrize("name,over,window,sinks", [
    ("C5", dict(batch=2, ctx=(3000, 2999)), 1000, 4),
    ("C5", dict(batch=2, ctx=(1500, 33)), 17, 5),
    ("C4", dict(batch=5, ctx=("uniform", 1, 700), extra_blocks=4), 100, 16),
    ("C3", dict(batch=2, ctx=(300, 40), capacity=300), 1, 0),
], ids=["C5-W1000", "C5-W17", "C4-W100", "C3-W1"])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_windowed_weights_match_oracle(name, over, window, sinks, num_splits):
    require_gpu()
    spec = W.preset(name, window=window, num_sinks=sinks, **over)
    announce(f"scores window {name} {over} W={window} n={sinks} S={num_splits}")
    w = W.make_workload(spec, device="cuda")
    _, scores = _run_scores(w, num_splits=num_splits)
    check_close(scores.cpu().numpy(), _oracle_scores(w), f"scores W={window} S={num_splits}")


def test_accumulate_adds_exactly_and_leaves_unattended_entries():
    require_gpu()
    spec = W.preset("C5", batch=2, ctx=(1500, 600), window=200, num_sinks=4)
    w = W.make_workload(spec, device="cuda")
    _, once = _run_scores(w)
    K = require_gpu()
    out = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")
    acc = torch.full_like(once, 7.0)
    call = K.decode_call_for(w, out, with_scores=True)
    call.decode_scores(acc, accumulate=True)
    call.decode_scores(acc, accumulate=True)
    torch.cuda.synchronize()
    attended = once > 0
    assert torch.equal(acc[attended], 7.0 + once[attended] + once[attended])
    assert (acc[~attended] == 7.0).all()


def test_scores_reject_several_query_tokens_and_missing_outputs():
    K = require_gpu()
    mixed = W.make_workload(W.preset("C1", batch=2, ctx=(256, 100), kv_dtype="bf16"), device="cuda")
    with pytest.raises(K.KvAttnError):  # score export takes bf16/bf16 or fp32/fp32 only
        _run_scores(mixed)
    spec = W.preset("C3", batch=2, ctx=(100, 50), capacity=100, num_queries=2)
    w = W.make_workload(spec, device="cuda")
    out = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")
    with pytest.raises(K.KvAttnError):
        K.decode_call_for(w, out, with_scores=True)
    spec1 = W.preset("C3", batch=2, ctx=(100, 50), capacity=100)
    w1 = W.make_workload(spec1, device="cuda")
    call = K.decode_call_for(w1, torch.empty(w1.q.shape, dtype=torch.float32, device="cuda"))
    import ctypes
    st = K._lib.kv_attn_decode_scores(*call._ptrs, None, 0, ctypes.byref(call.params), *call._ws, None)
    assert st == K.KV_ATTN_ERR_NULL
    st = K._lib.kv_attn_decode_scores(*call._ptrs, w1.q.data_ptr(), 0, ctypes.byref(call.params),
                                      None, 0, None)
    assert st == K.KV_ATTN_ERR_WORKSPACE


@pytest.mark.parametrize("name,seqs,heads", [("C5", [0, 3], [0, 5]), ("C4", "extremes", [0, 7]),
                                             ("C3", [0, 63], [1, 6])], ids=["C5", "C4", "C3"])
def test_full_size_weights_on_sampled_rows(name, seqs, heads):
    require_gpu()
    announce(f"scores full {name}")
    w = W.make_workload(W.PRESETS[name], device="cuda")
    try:
        _, scores = _run_scores(w)
        assert torch.isfinite(scores).all()
        if seqs == "extremes":
            order = np.argsort(w.ctx_lens.cpu().numpy(), kind="stable")
            seqs = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
        got = scores[seqs][:, heads].cpu().numpy()
        check_close(got, _oracle_scores(w, seqs, heads), f"scores full {name} seqs={seqs}")
    finally:
        del w
        torch.cuda.empty_cache()


def test_decode_scores_then_eviction_selects_what_the_oracle_selects():
    """Several layers of one sequence: export each layer's weights, then choose the entries that
    stay under a global budget on the GPU; the oracle selection over the same scores agrees bit
    for bit, and the weights agree with the oracle's."""
    require_gpu()
    from kv_cache_decode_split_amd import kv_evict
    from oracle import evict_select
    layers, T = 4, 2000
    spec = W.preset("C5", batch=1, ctx=(T,), layers=layers)
    per_layer = []
    for layer in range(layers):
        w = W.make_workload(spec, device="cuda", layer=layer)
        _, s = _run_scores(w)
        check_close(s.cpu().numpy(), _oracle_scores(w), f"pipeline layer {layer}")
        per_layer.append(s[0])
    scores = torch.stack(per_layer).contiguous()          # [L, h_kv, T]
    budget = layers * spec.num_kv_heads * T // 5
    keep = kv_evict.kv_evict_select(scores, budget)
    torch.cuda.synchronize()
    want = evict_select(scores.cpu().numpy(), budget)
    assert np.array_equal(keep.cpu().numpy().astype(bool), want)
    assert int(keep.sum()) == budget


def _random_score_specs(n, seed=31):
    import random
    rnd = random.Random(seed)
    specs = []
    for i in range(n):
        g = rnd.choice([1, 2, 4, 5, 8, 16])
        hkv = rnd.choice([1, 2, 3])
        B = rnd.randint(1, 3)
        paged = rnd.random() < 0.5
        lens = tuple(rnd.randint(0 if rnd.random() < 0.1 else 1, 2500) for _ in range(B))
        if max(lens) == 0:
            lens = (1,) + lens[1:]
        dt = rnd.choice(["bf16", "bf16", "f32"])
        specs.append(dict(
            spec=W.WorkloadSpec(
                name=f"rsc{i}", batch=B, num_q_heads=g * hkv, num_kv_heads=hkv,
                head_dim=rnd.choice([64, 128]), ctx=lens, paged=paged,
                block_size=rnd.choice([16, 32]) if paged else 16, kv_dtype=dt, q_dtype=dt,
                q_std=rnd.choice([1.0, 3.0]), num_sinks=rnd.choice([0, 4]),
                window=rnd.choice([None, None, 64, 700]),
                layout=rnd.choice(["head_major", "token_major"]), seed=11000 + i,
                capacity=None if paged else max(lens) + 3),
            num_splits=rnd.choice([0, 0, 1, 2, 5])))
    return specs


RANDOM = _random_score_specs(24)


@pytest.mark.parametrize("case", RANDOM, ids=[c["spec"].name for c in RANDOM])
def test_random_shapes_export_oracle_weights(case):
    require_gpu()
    spec = case["spec"]
    announce(f"scores random {spec} num_splits={case['num_splits']}")
    w = W.make_workload(spec, device="cuda")
    out, scores = _run_scores(w, num_splits=case["num_splits"])
    check_close(scores.cpu().numpy(), _oracle_scores(w), f"{spec.name} scores")
    _check_output(out, w, case["num_splits"], spec.name)
