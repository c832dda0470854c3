"""Seeded input generators: reproducibility, structure, poisoning (CPU only)."""

import numpy as np
import pytest
import torch

from kv_cache_decode_split_amd import workloads as W


def _small(name, **kw):
    base = dict(C4=dict(batch=6, ctx=("uniform", 1, 90)),
                C5=dict(batch=2, ctx=(70, 33)),
                C3=dict(batch=3, ctx=(50,) * 3),
                C2=dict(batch=2, ctx=(40, 40)),
                C1=dict())[name]
    base.update(kw)
    return W.preset(name, **base)


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5"])
def test_same_seed_same_bytes(name):
    a = W.make_workload(_small(name))
    b = W.make_workload(_small(name))
    for x, y in [(a.q, b.q), (a.k_cache, b.k_cache), (a.v_cache, b.v_cache), (a.ctx_lens, b.ctx_lens)]:
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.int32 else x,
                           y.view(torch.uint8) if y.dtype != torch.int32 else y)
    c = W.make_workload(_small(name), layer=1)
    assert not torch.equal(a.k_cache.nan_to_num(), c.k_cache.nan_to_num())


def test_presets_match_the_stated_shapes():
    p = W.PRESETS
    assert (p["C1"].batch, p["C1"].num_q_heads, p["C1"].num_kv_heads, p["C1"].head_dim) == (1, 8, 8, 64)
    assert p["C1"].kv_dtype == "f32" and p["C1"].ctx == (256,)
    assert (p["C2"].batch, p["C2"].num_q_heads, p["C2"].head_dim, p["C2"].layers) == (8, 32, 128, 32)
    assert p["C3"].group == 4 and p["C3"].q_std == 3.0 and p["C3"].ctx[0] == 8192
    assert p["C4"].paged and p["C4"].block_size == 16 and p["C4"].ctx == ("uniform", 128, 32768)
    assert p["C5"].group == 8 and p["C5"].num_sinks == 4 and p["C5"].ctx[0] == 131072


def test_c4_full_structure():
    """The real C4 structure (no K/V values drawn): lengths in range, a permutation table."""
    st = W.workload_structure(W.PRESETS["C4"])
    ctx = st["ctx"].numpy()
    assert ctx.min() >= 128 and ctx.max() <= 32768 and len(ctx) == 128
    table = st["table"].numpy()
    nblk = (ctx + 15) // 16
    live = np.concatenate([table[b, :n] for b, n in enumerate(nblk)])
    assert len(live) == len(set(live.tolist())) == nblk.sum()
    assert live.min() >= 0 and live.max() < st["num_blocks"]
    assert st["num_blocks"] == nblk.sum() + 1
    for b, n in enumerate(nblk):
        assert np.all(table[b, n:] == st["unused_blocks"][0])
    # a random permutation is not the identity layout
    assert np.mean(np.diff(live) == 1) < 0.01


def test_sequential_block_order_gives_each_sequence_a_physical_run():
    st = W.workload_structure(W.preset("C4", block_order="sequential", extra_blocks=2))
    ctx = st["ctx"].numpy()
    table = st["table"].numpy()
    nblk = (ctx + 15) // 16
    live = np.concatenate([table[b, :n] for b, n in enumerate(nblk)])
    assert np.array_equal(live, np.arange(nblk.sum()))
    assert st["unused_blocks"] == [int(nblk.sum()), int(nblk.sum()) + 1]
    with pytest.raises(ValueError):
        W.workload_structure(W.preset("C4", block_order="shuffled"))


@pytest.mark.parametrize("order", ["random", "sequential"])
def test_paged_tails_and_unused_blocks_are_poisoned(order):
    w = W.make_workload(_small("C4", extra_blocks=3, block_order=order))
    view = W.oracle_view(w)
    k = view["k_cache"]
    bits = k.view(np.uint16) if k.dtype == np.uint16 else None
    isnan = lambda a: (a & 0x7FFF) > 0x7F80  # noqa: E731  bf16 NaN patterns
    table, ctx, bs = view["block_table"], view["ctx_lens"], view["block_size"]
    live = set()
    for b, length in enumerate(ctx):
        n = (length + bs - 1) // bs
        for j in range(n):
            blk = table[b, j]
            live.add(int(blk))
            used = min(bs, length - j * bs)
            assert not isnan(bits[blk, :used]).any()
            assert isnan(bits[blk, used:]).all()
    for blk in range(w.num_blocks):
        if blk not in live:
            assert isnan(bits[blk]).all()


def test_contiguous_tails_are_poisoned():
    w = W.make_workload(W.preset("C3", batch=2, ctx=(20, 31), capacity=40))
    view = W.oracle_view(w)
    bits = view["k_cache"]
    isnan = lambda a: (a & 0x7FFF) > 0x7F80  # noqa: E731
    assert isnan(bits[0, 20:]).all() and not isnan(bits[0, :20]).any()
    assert isnan(bits[1, 31:]).all() and not isnan(bits[1, :31]).any()


def test_sinks_scale_the_first_keys_by_four():
    with_sinks = W.make_workload(_small("C5"))
    without = W.make_workload(_small("C5", num_sinks=0))
    a, b = W.oracle_view(with_sinks), W.oracle_view(without)
    widen = lambda u: (u.astype(np.uint32) << 16).view(np.float32)  # noqa: E731
    table, bs = a["block_table"], a["block_size"]
    for s in range(2):
        for t in range(6):
            blk, slot = table[s, t // bs], t % bs
            ka, kb = widen(a["k_cache"][blk, slot]), widen(b["k_cache"][blk, slot])
            if t < 4:
                assert np.array_equal(ka, kb * 4)
            else:
                assert np.array_equal(ka, kb)
    assert np.array_equal(a["v_cache"], b["v_cache"])


def test_query_spread_of_c3():
    w = W.make_workload(W.preset("C3", batch=64, ctx=(16,) * 64))
    assert abs(float(w.q.float().std()) - 3.0) < 0.05


def test_layouts_describe_the_same_logical_cache():
    hm = W.make_workload(_small("C4", layout="head_major"))
    tm = W.make_workload(_small("C4", layout="token_major"))
    assert hm.k_cache.shape[1:] == (8, 16, 128) and tm.k_cache.shape[1:] == (16, 8, 128)
    (ks, _), _ = hm.kv_strides(), None
    assert ks == (8 * 16 * 128, 128, 16 * 128)
    (kt, _) = tm.kv_strides()
    assert kt == (8 * 16 * 128, 8 * 128, 128)


def test_oracle_sample_renumbers_blocks():
    w = W.make_workload(_small("C4"))
    full = W.oracle_view(w)
    part = W.oracle_sample(w, [4, 1])
    bs = full["block_size"]
    for i, s in enumerate([4, 1]):
        n = (full["ctx_lens"][s] + bs - 1) // bs
        assert part["ctx_lens"][i] == full["ctx_lens"][s]
        assert np.array_equal(part["q"][i], full["q"][s])
        for j in range(n):
            a = part["k_cache"][part["block_table"][i, j]]
            b = full["k_cache"][full["block_table"][s, j]]
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("paged,layout", [(True, "head_major"), (True, "token_major"),
                                          (False, "head_major"), (False, "token_major")])
def test_window_poisons_exactly_the_unattended_positions(paged, layout):
    """With a window, every position outside the first num_sinks and the last W positions holds
    NaN in K and V; every attended position holds the same finite value as without a window."""
    from oracle import attended_positions, decode_attention
    ctx = (200, 37, 96, 5)
    kw = dict(batch=4, ctx=ctx, paged=paged, layout=layout, num_sinks=3, block_size=16,
              capacity=None if paged else 210)
    plain = W.make_workload(W.preset("C5", **kw))
    win = W.make_workload(W.preset("C5", window=40, **kw))
    a, b = W.oracle_view(plain), W.oracle_view(win)
    isnan = lambda u: (u & 0x7FFF) > 0x7F80  # noqa: E731
    for s, length in enumerate(ctx):
        keep = set(attended_positions(length, 40, 3).tolist())
        for t in range(length):
            if paged:
                blk, slot = a["block_table"][s, t // 16], t % 16
            else:
                blk, slot = s, t
            for name in ("k_cache", "v_cache"):
                x, y = a[name][blk, slot], b[name][blk, slot]
                if t in keep:
                    assert np.array_equal(x, y) and not isnan(y).any(), (s, t, name)
                else:
                    assert isnan(y).all(), (s, t, name)
    # The oracle never touches the poisoned rows: same result as over the clean cache.
    bs = a["block_size"] if paged else None
    ref = decode_attention(a["q"], a["k_cache"], a["v_cache"], a["ctx_lens"], a["block_table"],
                           block_size=bs, window=40, num_sinks=3)
    got = decode_attention(b["q"], b["k_cache"], b["v_cache"], b["ctx_lens"], b["block_table"],
                           block_size=bs, window=40, num_sinks=3)
    assert np.isfinite(got).all() and np.array_equal(ref, got)


@pytest.mark.parametrize("paged", [True, False])
def test_gamma_tokens_spare_the_union_of_their_windows(paged):
    """With gamma query tokens, q is [B, gamma, h_q, d] and the window poisoning spares every
    position some token attends (the union of the tokens' windows and the sinks)."""
    from oracle import attended_positions, verify_attention
    ctx, gamma, window, sinks = (200, 37, 3), 4, 30, 2
    kw = dict(batch=3, ctx=ctx, paged=paged, num_sinks=sinks, capacity=None if paged else 210)
    plain = W.make_workload(W.preset("C5", num_queries=gamma, **kw))
    win = W.make_workload(W.preset("C5", num_queries=gamma, window=window, **kw))
    assert tuple(win.q.shape) == (3, gamma, 64, 128)
    assert torch.equal(plain.q.view(torch.int16), win.q.view(torch.int16))
    a, b = W.oracle_view(plain), W.oracle_view(win)
    isnan = lambda u: (u & 0x7FFF) > 0x7F80  # noqa: E731
    for s, length in enumerate(ctx):
        keep = set()
        for j in range(gamma):
            visible = length - gamma + 1 + j
            if visible > 0:
                keep |= set(attended_positions(visible, window, sinks).tolist())
        for t in range(length):
            blk, slot = ((a["block_table"][s, t // 16], t % 16) if paged else (s, t))
            y = b["k_cache"][blk, slot]
            assert (not isnan(y).any()) if t in keep else isnan(y).all(), (s, t)
    bs = a["block_size"] if paged else None
    ref = verify_attention(a["q"], a["k_cache"], a["v_cache"], a["ctx_lens"], a["block_table"],
                           block_size=bs, window=window, num_sinks=sinks)
    got = verify_attention(b["q"], b["k_cache"], b["v_cache"], b["ctx_lens"], b["block_table"],
                           block_size=bs, window=window, num_sinks=sinks)
    assert np.isfinite(got).all() and np.array_equal(ref, got)


@pytest.mark.parametrize("kind", ["lognormal", "normal", "levels", "equal"])
def test_scores_are_seeded_and_strided_views_hide_their_padding(kind):
    a = W.make_scores(3, 4, 50, kind, seed=5)
    b = W.make_scores(3, 4, 50, kind, seed=5)
    assert a.shape == (3, 4, 50) and a.dtype == torch.float32 and a.is_contiguous()
    assert torch.equal(a, b)
    s = W.make_scores(3, 4, 50, kind, seed=5, row_stride=53)
    assert s.shape == (3, 4, 50) and s.stride() == (4 * 53, 53, 1)
    assert torch.isfinite(s).all()
    store = s.as_strided((12, 53), (53, 1))
    assert torch.isnan(store[:, 50:]).all()   # the padding is never meant to be read
    if kind == "lognormal":
        assert (a > 0).all()
    if kind == "levels":
        assert set(a.unique().tolist()) <= {0.0, 0.25, 0.5, 1.0}
    if kind == "equal":
        assert (a == 1.0).all()
