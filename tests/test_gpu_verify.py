"""GPU parity of γ-query verification decode (several query tokens per sequence) against the
fp64 oracle ``oracle.verify_attention``.

The γ query tokens of a sequence of length T are its last γ cached positions; token j sees the
first T - γ + 1 + j positions (a zero row when that is <= 0), with a window applied to its own
visible prefix. The caches are NaN-poisoned outside what some token may attend (past T, and with
a window outside the union of the tokens' windows and the sinks), so a finite output that
matches the oracle also shows that nothing else was read. Tolerance as for the other parity
tests; ``q_std`` 3 workloads (a peaked softmax) exercise the accuracy of P in the P.V product.
"""

import random

import numpy as np
import pytest
import torch

from kv_cache_decode_split_amd import workloads as W
from tests.gpu_helpers import announce, check_close, require_gpu, run

pytestmark = pytest.mark.gpu


def _window_kwargs(spec):
    return {} if spec.window is None else dict(window=spec.window, num_sinks=spec.num_sinks)


def oracle_verify(w, seqs=None, kv_heads=None):
    from oracle import verify_attention
    v = W.oracle_view(w) if seqs is None else W.oracle_sample(w, seqs, kv_heads)
    paged = v["block_table"] is not None
    return verify_attention(v["q"], v["k_cache"], v["v_cache"], v["ctx_lens"], v["block_table"],
                            block_size=v["block_size"] if paged else None,
                            **_window_kwargs(w.spec))


def select(out, w, seqs, kv_heads=None):
    o = out[[int(s) for s in seqs]]
    if kv_heads is not None:
        g = w.spec.group
        heads = [kvh * g + j for kvh in kv_heads for j in range(g)]
        o = o[:, :, heads]
    return o.cpu().numpy().astype(np.float64)


SMALL = [
    # (preset, overrides, gamma)
    ("C3", dict(batch=3, ctx=(1000, 77, 4), capacity=1010), 4),          # T == gamma
    ("C5", dict(batch=2, ctx=(3000, 1777)), 4),                           # 32 rows, two blocks
    ("C5", dict(batch=3, ctx=(2, 1, 0)), 2),                              # T < gamma, empty
    ("C2", dict(batch=4, ctx=(700, 15, 16, 17), layers=1), 16),           # 16 tokens, g = 1
    ("C4", dict(batch=6, ctx=("uniform", 1, 700), layout="token_major"), 8),
    ("C5", dict(batch=2, ctx=(900, 333), num_q_heads=16, num_kv_heads=2, head_dim=64), 3),
    ("C3", dict(batch=2, ctx=(513, 250), num_q_heads=10, num_kv_heads=2, capacity=520), 5),
    ("C4", dict(batch=4, ctx=("uniform", 200, 900), block_size=64), 2),
    ("C3", dict(batch=2, ctx=(4100, 4095), capacity=4100, q_std=3.0), 8),  # peaked softmax
]


@pytest.mark.parametrize("name,over,gamma", SMALL, ids=[f"{n}-g{g}-{i}" for i, (n, _, g) in enumerate(SMALL)])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_small_verification_workloads_match_oracle(name, over, gamma, num_splits):
    require_gpu()
    spec = W.preset(name, num_queries=gamma, **over)
    announce(f"verify {name} {over} gamma={gamma} num_splits={num_splits}")
    w = W.make_workload(spec, device="cuda")
    assert tuple(w.q.shape) == (spec.batch, gamma, spec.num_q_heads, spec.head_dim)
    out = run(w, num_splits=num_splits)
    check_close(out.cpu().numpy(), oracle_verify(w), f"verify {name} gamma={gamma} S={num_splits}")


WINDOWED = [
    # (preset, overrides, gamma, window, sinks)
    ("C5", dict(batch=2, ctx=(3000, 2999)), 4, 1000, 4),
    ("C5", dict(batch=2, ctx=(1500, 33)), 4, 17, 5),                  # edges inside tiles
    ("C3", dict(batch=2, ctx=(300, 40), capacity=300), 4, 1, 0),      # each token sees itself
    ("C4", dict(batch=5, ctx=("uniform", 1, 700), extra_blocks=4), 2, 100, 16),
    ("C2", dict(batch=2, ctx=(700, 20), layers=1), 16, 30, 3),         # window shorter than gamma
]


@pytest.mark.parametrize("name,over,gamma,window,sinks", WINDOWED,
                         ids=[f"{n}-g{g}-W{wd}" for n, _, g, wd, _ in WINDOWED])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_windowed_verification_matches_oracle(name, over, gamma, window, sinks, num_splits):
    require_gpu()
    spec = W.preset(name, num_queries=gamma, window=window, num_sinks=sinks, **over)
    announce(f"verify-window {name} {over} gamma={gamma} W={window} n={sinks} S={num_splits}")
    w = W.make_workload(spec, device="cuda")
    out = run(w, num_splits=num_splits)
    check_close(out.cpu().numpy(), oracle_verify(w),
                f"verify {name} gamma={gamma} W={window} S={num_splits}")


def _random_specs(n, seed=23):
    rnd = random.Random(seed)
    specs = []
    for i in range(n):
        g = rnd.choice([1, 2, 4, 5, 8, 16])
        gamma = rnd.choice([k for k in range(2, 17) if k * g <= 32])
        hkv = rnd.choice([1, 2, 3])
        B = rnd.randint(1, 4)
        paged = rnd.random() < 0.6
        lens = tuple(rnd.randint(0, 40) if rnd.random() < 0.2 else rnd.randint(1, 3000)
                     for _ in range(B))
        window = rnd.choice([None, None, 1, 16, 100, 700])
        specs.append(dict(
            spec=W.WorkloadSpec(
                name=f"rver{i}", batch=B, num_q_heads=g * hkv, num_kv_heads=hkv,
                head_dim=rnd.choice([64, 128]), ctx=lens, paged=paged,
                block_size=rnd.choice([16, 32, 128]) if paged else 16, q_std=rnd.choice([1.0, 3.0]),
                num_sinks=rnd.choice([0, 4, 37]), window=window, num_queries=gamma,
                layout=rnd.choice(["head_major", "token_major"]), seed=9000 + i,
                extra_blocks=rnd.randint(1, 3), capacity=None if paged else max(max(lens), 1) + 2),
            num_splits=rnd.choice([0, 0, 1, 2, 5])))
    return specs


RANDOM = _random_specs(24)


@pytest.mark.parametrize("case", RANDOM, ids=[c["spec"].name for c in RANDOM])
def test_random_verification_shapes_match_oracle(case):
    require_gpu()
    spec = case["spec"]
    announce(f"verify random {spec} num_splits={case['num_splits']}")
    w = W.make_workload(spec, device="cuda")
    out = run(w, num_splits=case["num_splits"])
    check_close(out.cpu().numpy(), oracle_verify(w), f"{spec.name}")


def test_gamma_one_tokens_equal_single_token_decode_bitwise():
    """num_queries = 1 is the single-token path: a [B, 1, h_q, d] q gives the same bits."""
    require_gpu()
    spec = W.preset("C5", batch=2, ctx=(2000, 555))
    w = W.make_workload(spec, device="cuda")
    base = run(w)
    w.q = w.q[:, None].contiguous()
    one = run(w)
    assert torch.equal(one[:, 0], base)


def test_verification_rows_match_decode_of_shorter_contexts():
    """Token j of a draft of gamma is a single-token decode over the first T - gamma + 1 + j
    positions: both GPU paths agree with each other to the parity tolerance."""
    K = require_gpu()
    gamma, T = 4, 1500
    spec = W.preset("C3", batch=1, ctx=(T,), capacity=T, num_queries=gamma)
    w = W.make_workload(spec, device="cuda")
    out = run(w)
    for j in range(gamma):
        ref = torch.full((1, spec.num_q_heads, spec.head_dim), float("nan"), device="cuda")
        lens = torch.tensor([T - gamma + 1 + j], dtype=torch.int32, device="cuda")
        ks, vs = w.kv_strides()
        K.kv_attn_decode(w.q[:, j].contiguous(), w.k_cache, w.v_cache, None, lens, ref,
                         num_kv_heads=spec.num_kv_heads, k_strides=ks, v_strides=vs,
                         block_size=w.block_size, num_blocks=w.num_blocks, max_ctx_len=T)
        torch.cuda.synchronize()
        check_close(out[:, j].cpu().numpy(), ref.cpu().numpy(), f"token {j}")


FULL = [
    # (preset, gamma, sampled sequences, sampled KV heads)
    ("C3", 4, [0, 63], [0, 7]),
    ("C5", 4, [0, 3], [0, 5]),
    ("C4", 2, "extremes", [0, 7]),
]


@pytest.mark.parametrize("name,gamma,seqs,heads", FULL, ids=[f"{n}-g{g}" for n, g, _, _ in FULL])
def test_full_size_verification_on_sampled_rows(name, gamma, seqs, heads):
    """Full-size workloads with gamma query tokens (auto split plan); sampled rows checked."""
    require_gpu()
    announce(f"verify full {name} gamma={gamma}")
    w = W.make_workload(W.preset(name, num_queries=gamma), device="cuda")
    try:
        out = run(w)
        assert torch.isfinite(out).all(), "non-finite output somewhere in the full batch"
        if seqs == "extremes":
            order = np.argsort(w.ctx_lens.cpu().numpy(), kind="stable")
            seqs = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
        check_close(select(out, w, seqs, heads), oracle_verify(w, seqs, heads),
                    f"verify full {name} gamma={gamma} seqs={seqs}")
    finally:
        del w
        torch.cuda.empty_cache()


def _np_rows(t):
    t = t.cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _poison_last(w, n):
    """NaN at the last n positions of every sequence: only a real append makes them readable."""
    bt = None if w.block_table is None else w.block_table.cpu()
    kv = w.k_cache.permute(0, 2, 1, 3) if w.spec.layout == "head_major" else w.k_cache
    vv = w.v_cache.permute(0, 2, 1, 3) if w.spec.layout == "head_major" else w.v_cache
    for b, t in enumerate(w.ctx_lens.cpu().tolist()):
        for p in range(max(t - n, 0), t):
            blk, slot = (b, p) if bt is None else (int(bt[b, p // w.block_size]), p % w.block_size)
            kv[blk, slot].fill_(float("nan"))
            vv[blk, slot].fill_(float("nan"))


@pytest.mark.parametrize("name,over,gamma", [
    ("C4", dict(batch=5, ctx=("uniform", 4, 900)), 4),
    ("C3", dict(batch=3, ctx=(100, 8, 40), capacity=100, layout="token_major"), 8),
], ids=["C4-g4", "C3-g8"])
def test_append_decode_with_gamma_tokens_matches_oracle(name, over, gamma):
    """The gamma draft rows are appended at T - gamma .. T - 1 and then verified in one call."""
    K = require_gpu()
    from oracle import append_kv, verify_attention
    spec = W.preset(name, num_queries=gamma, **over)
    announce(f"verify append_decode {name} {over} gamma={gamma}")
    w = W.make_workload(spec, device="cuda")
    _poison_last(w, gamma)
    before = W.oracle_view(w)
    gen = torch.Generator(device="cpu").manual_seed(5)
    shape = (spec.batch, gamma, spec.num_kv_heads, spec.head_dim)
    k_new = torch.randn(shape, generator=gen).to(w.k_cache.dtype).cuda()
    v_new = torch.randn(shape, generator=gen).to(w.v_cache.dtype).cuda()
    out = torch.full(w.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    K.decode_call_for(w, out).append_decode(k_new, v_new)
    torch.cuda.synchronize()
    pos = before["ctx_lens"] - gamma
    table = before["block_table"]
    kw = dict(block_size=w.block_size) if table is not None else dict(capacity=w.block_size)
    kc = append_kv(before["k_cache"], _np_rows(k_new), pos, table, **kw)
    vc = append_kv(before["v_cache"], _np_rows(v_new), pos, table, **kw)
    ref = verify_attention(before["q"], kc, vc, before["ctx_lens"], table,
                           block_size=w.block_size if table is not None else None)
    check_close(out.cpu().numpy(), ref, f"verify append_decode {name} gamma={gamma}")


def test_append_of_several_tokens_matches_oracle_bitwise():
    K = require_gpu()
    from oracle import append_kv
    spec = W.preset("C4", batch=4, ctx=("uniform", 20, 300))
    w = W.make_workload(spec, device="cuda")
    before = W.oracle_view(w)
    n = 5
    gen = torch.Generator(device="cpu").manual_seed(9)
    shape = (spec.batch, n, spec.num_kv_heads, spec.head_dim)
    k_new = torch.randn(shape, generator=gen).to(w.k_cache.dtype).cuda()
    v_new = torch.randn(shape, generator=gen).to(w.v_cache.dtype).cuda()
    cap = w.block_table.shape[1] * w.block_size
    pos = np.array([0, cap - 2, -1, 7], dtype=np.int32)  # a run cut by the capacity, an idle one
    ks, vs = w.kv_strides()
    K.kv_attn_append(k_new, v_new, w.k_cache, w.v_cache, w.block_table,
                     torch.from_numpy(pos).cuda(), num_kv_heads=spec.num_kv_heads, k_strides=ks,
                     v_strides=vs, block_size=w.block_size, num_blocks=w.num_blocks)
    torch.cuda.synchronize()
    after = W.oracle_view(w)
    for name, new in (("k_cache", k_new), ("v_cache", v_new)):
        want = append_kv(before[name], _np_rows(new), pos, before["block_table"],
                         block_size=w.block_size)
        got = np.ascontiguousarray(after[name])
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), name
