"""Seeded synthetic inputs for decode attention.

This module is the only code that both the oracle side (tests, bench CPU baseline) and the HIP
side use. It holds none of the method's arithmetic: it draws random numbers, rounds the draws
to the storage type, lays the cache out in memory, builds block tables and context lengths, and
poisons with NaN every slot the attention must never read. Nothing here computes scores,
softmax or weighted sums.

Workload shapes follow the examples the pages reason about (no dataset is involved):

* C1: one layer, MHA, B=1, h_q=h_kv=8, d=64, T=256, fp32 q/K/V ~ N(0,1), contiguous.
* C2: LLaMA-7B-shaped layer (Ch. 19 §19.3.2 and §19.4.2 size the 7B model at 32 layers and
  hidden 4096): B=8, h_q=h_kv=32, d=128, T=4096, bf16 q/K/V ~ N(0,1), contiguous; a decode step
  runs 32 such layers, each with its own cache.
* C3: GQA group 4: B=64, h_q=32, h_kv=8, d=128, T=8192, bf16 K/V ~ N(0,1), q ~ N(0, 3^2) so that
  the score spread is about 3 (a peaked softmax).
* C4: paged GQA (Ch. 19 §19.7.3, 16-token blocks): B=128, h_q=32, h_kv=8, d=128, context lengths
  uniform integers in [128, 32768], block table a random permutation of the physical blocks.
* C5: long-context split-KV: B=4, h_q=64, h_kv=8 (group 8), d=128, T=131072, paged 16-token
  blocks, and 4 "sink" positions (StreamingLLM's attention sinks, Ch. 19 §19.4.3) at the start of
  every sequence whose key rows are scaled by 4.

Cache layouts (both are described to the library by element strides):

* ``head_major`` (default): paged ``[num_blocks, h_kv, block_size, d]``, contiguous
  ``[B, h_kv, capacity, d]``. The rows one (sequence, KV head) pair streams are adjacent.
* ``token_major``: paged ``[num_blocks, block_size, h_kv, d]``, contiguous
  ``[B, capacity, h_kv, d]``.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

__all__ = [
    "WorkloadSpec",
    "Workload",
    "PRESETS",
    "preset",
    "make_workload",
    "workload_structure",
    "oracle_view",
    "oracle_sample",
    "EVICT_PRESETS",
    "make_scores",
]

# Elements per random draw; fixed so that a seed gives the same bytes on every run.
_CHUNK = 1 << 24


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    # Either an explicit tuple of per-sequence lengths, or ("uniform", lo, hi) inclusive.
    ctx: tuple
    paged: bool = False
    block_size: int = 16
    kv_dtype: str = "bf16"          # "bf16" | "f32"
    q_dtype: str = "bf16"           # "bf16" | "f32"
    q_std: float = 1.0
    num_sinks: int = 0
    sink_scale: float = 4.0
    layout: str = "head_major"      # "head_major" | "token_major"
    seed: int = 0
    layers: int = 1
    extra_blocks: int = 1           # paged: unused (NaN) physical blocks, at least 1
    capacity: Optional[int] = None  # contiguous: tokens per sequence slot (default max ctx)
    # Sliding window: None attends every position; W >= 1 attends only the first num_sinks and
    # the last W positions of each sequence, and every other position is NaN-poisoned.
    window: Optional[int] = None
    # Query tokens per sequence (gamma). gamma > 1: q is [B, gamma, h_q, d] and the tokens are
    # the last gamma cached positions (a speculative draft being checked); the window poisoning
    # then spares the union of the gamma tokens' windows.
    num_queries: int = 1
    # Paged: "random" deals the physical blocks to the sequences in a seeded random order;
    # "sequential" gives every sequence a run of consecutive physical blocks, as a fresh
    # allocator hands them out.
    block_order: str = "random"
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


PRESETS = {
    "C1": WorkloadSpec(
        name="C1", batch=1, num_q_heads=8, num_kv_heads=8, head_dim=64, ctx=(256,),
        kv_dtype="f32", q_dtype="f32", seed=1001,
        description="single-layer MHA decode attention, B=1, h_q=h_kv=8, d=64, T=256, fp32 "
                    "q/K/V ~ N(0,1), contiguous KV, fp32 output"),
    "C2": WorkloadSpec(
        name="C2", batch=8, num_q_heads=32, num_kv_heads=32, head_dim=128, ctx=(4096,) * 8,
        seed=1002, layers=32,
        description="LLaMA-7B-shaped layer decode attention, B=8, h_q=h_kv=32, d=128, T=4096, "
                    "bf16 q/K/V ~ N(0,1), contiguous KV, 32 layers = 32 launches per step"),
    "C3": WorkloadSpec(
        name="C3", batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128, ctx=(8192,) * 64,
        q_std=3.0, seed=1003,
        description="GQA decode attention, B=64, h_q=32, h_kv=8 (group 4), d=128, T=8192, bf16 "
                    "K/V ~ N(0,1), q ~ N(0,9) (score spread ~3), contiguous KV"),
    "C4": WorkloadSpec(
        name="C4", batch=128, num_q_heads=32, num_kv_heads=8, head_dim=128,
        ctx=("uniform", 128, 32768), paged=True, block_size=16, seed=1004,
        description="paged GQA decode attention, B=128, h_q=32, h_kv=8, d=128, 16-token "
                    "blocks, random-permutation block table, T ~ U{128..32768}, bf16"),
    "C5": WorkloadSpec(
        name="C5", batch=4, num_q_heads=64, num_kv_heads=8, head_dim=128, ctx=(131072,) * 4,
        paged=True, block_size=16, num_sinks=4, seed=1005,
        description="long-context split-KV decode attention, B=4, h_q=64, h_kv=8 (group 8), "
                    "d=128, T=131072, 16-token paged blocks, 4 sink keys scaled x4, bf16"),
}


def preset(name: str, **overrides) -> WorkloadSpec:
    """A named preset, optionally with fields replaced (e.g. a shorter context for tests)."""
    return dataclasses.replace(PRESETS[name], **overrides)


@dataclasses.dataclass
class Workload:
    spec: WorkloadSpec
    q: torch.Tensor                       # [B, h_q, d], or [B, gamma, h_q, d] when gamma > 1
    k_cache: torch.Tensor                 # storage tensor (layout per spec.layout)
    v_cache: torch.Tensor
    block_table: Optional[torch.Tensor]   # int32 [B, max_blocks] or None (contiguous)
    ctx_lens: torch.Tensor                # int32 [B]
    block_size: int                       # tokens per block (paged) or capacity (contiguous)
    num_blocks: int                       # physical blocks (contiguous: B)
    layer: int = 0

    @property
    def max_ctx_len(self) -> int:
        return int(self.ctx_lens.max().item()) if self.ctx_lens.numel() else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1]) if self.block_table is not None else 1

    def kv_strides(self):
        """Element strides (block, token, head) of the K and V caches; the dim stride is 1."""
        def strides(t):
            s = t.stride()
            if self.spec.layout == "head_major":
                return (s[0], s[2], s[1])
            return (s[0], s[1], s[2])
        return strides(self.k_cache), strides(self.v_cache)


def _dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def _generator(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + stream * 7919) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def _fill_normal(out: torch.Tensor, gen: torch.Generator, std: float) -> None:
    """Fill ``out`` (contiguous) with N(0, std^2) draws rounded to its dtype, chunk by chunk."""
    flat = out.view(-1)
    n = flat.numel()
    for start in range(0, n, _CHUNK):
        stop = min(n, start + _CHUNK)
        draw = torch.randn(stop - start, generator=gen, device=out.device, dtype=torch.float32)
        if std != 1.0:
            draw.mul_(std)
        flat[start:stop].copy_(draw)  # rounds to nearest even for bf16


def _ctx_lens(spec: WorkloadSpec) -> torch.Tensor:
    if len(spec.ctx) == 3 and spec.ctx[0] == "uniform":
        _, lo, hi = spec.ctx
        g = _generator(spec.seed, 1, "cpu")
        return torch.randint(int(lo), int(hi) + 1, (spec.batch,), generator=g, dtype=torch.int64).to(torch.int32)
    if len(spec.ctx) != spec.batch:
        raise ValueError(f"{spec.name}: {len(spec.ctx)} context lengths for batch {spec.batch}")
    return torch.tensor([int(t) for t in spec.ctx], dtype=torch.int32)


def workload_structure(spec: WorkloadSpec, layer: int = 0) -> dict:
    """Context lengths, block table and storage shape of ``spec`` (no K/V values), on the CPU.

    Paged caches: every sequence gets ceil(T_b / block_size) physical blocks, taken in order
    from a seeded random permutation of all physical blocks (``block_order="sequential"``: from
    the blocks in physical order); the blocks left over (at least one)
    are never referenced by a live table entry, and table entries past a sequence's last block
    point at one of them (it is NaN-poisoned, so a stray read shows up in the output).
    """
    if spec.num_q_heads % spec.num_kv_heads:
        raise ValueError("h_q must be a multiple of h_kv")
    seed = spec.seed + 7919 * layer
    ctx = _ctx_lens(spec)
    B, hkv, d = spec.batch, spec.num_kv_heads, spec.head_dim
    if spec.paged:
        bs = spec.block_size
        if bs < 16 or bs & (bs - 1):
            raise ValueError("paged block_size must be a power of two >= 16")
        nblk = [(int(t) + bs - 1) // bs for t in ctx.tolist()]
        used = sum(nblk)
        total = used + max(1, spec.extra_blocks)
        if spec.block_order == "random":
            perm = torch.randperm(total, generator=_generator(seed, 3, "cpu")).to(torch.int32)
        elif spec.block_order == "sequential":
            perm = torch.arange(total, dtype=torch.int32)
        else:
            raise ValueError(f"block_order {spec.block_order!r}")
        poison_block = int(perm[used].item())
        table = torch.full((B, max(1, max(nblk))), poison_block, dtype=torch.int32)
        off = 0
        for b, n in enumerate(nblk):
            table[b, :n] = perm[off:off + n]
            off += n
        shape = (total, hkv, bs, d) if spec.layout == "head_major" else (total, bs, hkv, d)
        return dict(ctx=ctx, table=table, block_size=bs, num_blocks=total,
                    unused_blocks=perm[used:].tolist(), shape=shape)
    cap = spec.capacity if spec.capacity is not None else max(1, int(ctx.max().item()))
    if int(ctx.max().item()) > cap:
        raise ValueError("context longer than the contiguous capacity")
    shape = (B, hkv, cap, d) if spec.layout == "head_major" else (B, cap, hkv, d)
    return dict(ctx=ctx, table=None, block_size=cap, num_blocks=B, unused_blocks=[], shape=shape)


def make_workload(spec: WorkloadSpec, device="cpu", layer: int = 0) -> Workload:
    """Build the seeded inputs of ``spec`` on ``device``.

    The structure (context lengths, block table) is always drawn on the CPU, so it is identical
    whichever device holds the tensors. q/K/V draws use a generator on ``device``; layer ``l`` of
    a multi-layer spec uses its own seed stream.
    """
    device = torch.device(device)
    st = workload_structure(spec, layer)
    seed = spec.seed + 7919 * layer
    ctx, table, shape = st["ctx"], st["table"], st["shape"]
    block_size, num_blocks = st["block_size"], st["num_blocks"]
    B, hq, d = spec.batch, spec.num_q_heads, spec.head_dim
    kv_dt, q_dt = _dtype(spec.kv_dtype), _dtype(spec.q_dtype)

    q_shape = (B, hq, d) if spec.num_queries <= 1 else (B, spec.num_queries, hq, d)
    q = torch.empty(q_shape, dtype=q_dt, device=device)
    _fill_normal(q, _generator(seed, 2, device), spec.q_std)

    k = torch.empty(shape, dtype=kv_dt, device=device)
    v = torch.empty(shape, dtype=kv_dt, device=device)
    _fill_normal(k, _generator(seed, 4, device), 1.0)
    _fill_normal(v, _generator(seed, 5, device), 1.0)

    def bshd(t):  # view with axes [block, slot, head, dim]
        return t.permute(0, 2, 1, 3) if spec.layout == "head_major" else t

    kv, vv = bshd(k), bshd(v)
    ctx_list = ctx.tolist()
    nan = float("nan")
    for b, length in enumerate(ctx_list):
        if table is None:
            blk_of = lambda t, b=b: (b, t)  # noqa: E731
        else:
            blk_of = lambda t, b=b: (int(table[b, t // block_size]), t % block_size)  # noqa: E731
        # Attention sinks: the first positions of every sequence get larger keys. Scaling by a
        # power of two commutes with rounding, so this equals scaling before rounding.
        for t in range(min(spec.num_sinks, length)):
            blk, slot = blk_of(t)
            kv[blk, slot].mul_(spec.sink_scale)
        # Poison the slots past the end of the sequence inside its last block / slot range.
        if table is None:
            if length < block_size:
                kv[b, length:].fill_(nan)
                vv[b, length:].fill_(nan)
        elif length % block_size:
            blk, slot = blk_of(length - 1)
            kv[blk, slot + 1:].fill_(nan)
            vv[blk, slot + 1:].fill_(nan)
    for blk in st["unused_blocks"]:
        kv[blk].fill_(nan)
        vv[blk].fill_(nan)
    if spec.window is not None:
        _poison_outside_window(k, v, kv, vv, spec, ctx_list, table, block_size)

    ctx_dev = ctx.to(device)
    table_dev = table.to(device) if table is not None else None
    return Workload(spec=spec, q=q, k_cache=k, v_cache=v, block_table=table_dev, ctx_lens=ctx_dev,
                    block_size=block_size, num_blocks=num_blocks, layer=layer)


def _poison_outside_window(k, v, kv, vv, spec, ctx_list, table, block_size) -> None:
    """NaN into every position of a windowed sequence that is neither one of its first
    ``num_sinks`` positions nor one of its last ``window`` positions (with gamma query tokens,
    the last ``window + gamma - 1``). Whole blocks of such positions are filled with one indexed
    fill; the (at most two) blocks cut by an edge slot by slot range."""
    nan = float("nan")
    whole = []
    span = spec.window + max(spec.num_queries, 1) - 1
    for b, length in enumerate(ctx_list):
        lo, hi = min(spec.num_sinks, length), max(length - span, 0)  # gap [lo, hi)
        if hi <= lo:
            continue
        if table is None:
            kv[b, lo:hi].fill_(nan)
            vv[b, lo:hi].fill_(nan)
            continue
        for j in range(lo // block_size, (hi + block_size - 1) // block_size):
            start = j * block_size
            a, e = max(lo, start), min(hi, start + block_size)
            blk = int(table[b, j])
            if a == start and e == start + block_size:
                whole.append(blk)
            else:
                kv[blk, a - start:e - start].fill_(nan)
                vv[blk, a - start:e - start].fill_(nan)
    if whole:
        idx = torch.tensor(whole, dtype=torch.int64, device=k.device)
        k.index_fill_(0, idx, nan)  # axis 0 is the physical block in both layouts
        v.index_fill_(0, idx, nan)


def _np_storage(t: torch.Tensor) -> np.ndarray:
    """A host numpy view of a tensor's stored values: float32 as is, bf16 as uint16 bits."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


def oracle_view(w: Workload) -> dict:
    """All inputs as host numpy arrays in the oracle's conventions (whole workload)."""
    def bshd(t):
        a = _np_storage(t)
        return a.transpose(0, 2, 1, 3) if w.spec.layout == "head_major" else a
    return dict(
        q=_np_storage(w.q), k_cache=bshd(w.k_cache), v_cache=bshd(w.v_cache),
        ctx_lens=w.ctx_lens.cpu().numpy().astype(np.int64),
        block_table=None if w.block_table is None else w.block_table.cpu().numpy().astype(np.int64),
        block_size=w.block_size,
    )


def oracle_sample(w: Workload, seqs, kv_heads=None) -> dict:
    """Host copy of only the sequences ``seqs`` (and optionally only the KV heads ``kv_heads``
    with their query heads), in the oracle's conventions.

    The physical blocks a sampled sequence uses are copied (nothing else), and the block table
    is renumbered to the copy. Oracle output rows correspond to ``seqs`` in order, and its head
    axis to the query heads of ``kv_heads`` in order.
    """
    seqs = [int(s) for s in seqs]
    ctx = w.ctx_lens.cpu().to(torch.int64)
    q_sel = w.q[seqs]
    if kv_heads is not None:
        g = w.spec.group
        heads = [kvh * g + j for kvh in kv_heads for j in range(g)]
        q_sel = q_sel[:, heads] if q_sel.dim() == 3 else q_sel[:, :, heads]
    q = _np_storage(q_sel)
    if w.block_table is None:
        idx = torch.tensor(seqs, dtype=torch.int64, device=w.k_cache.device)
        k = w.k_cache.index_select(0, idx)
        v = w.v_cache.index_select(0, idx)
        table = None
    else:
        bs = w.block_size
        rows, phys, count = [], [], 0
        for s in seqs:
            n = (int(ctx[s]) + bs - 1) // bs
            phys.append(w.block_table[s, :n].to(torch.int64))
            rows.append(list(range(count, count + n)))
            count += n
        idx = torch.cat(phys) if phys else torch.zeros(0, dtype=torch.int64, device=w.k_cache.device)
        k = w.k_cache.index_select(0, idx)
        v = w.v_cache.index_select(0, idx)
        width = max(1, max(len(r) for r in rows))
        table = np.zeros((len(seqs), width), dtype=np.int64)
        for i, r in enumerate(rows):
            table[i, :len(r)] = r

    if kv_heads is not None:
        axis = 1 if w.spec.layout == "head_major" else 2
        hidx = torch.tensor([int(h) for h in kv_heads], dtype=torch.int64, device=k.device)
        k = k.index_select(axis, hidx)
        v = v.index_select(axis, hidx)

    def bshd(t):
        a = _np_storage(t)
        return a.transpose(0, 2, 1, 3) if w.spec.layout == "head_major" else a
    return dict(q=q, k_cache=bshd(k), v_cache=bshd(v),
                ctx_lens=ctx[seqs].numpy().astype(np.int64), block_table=table,
                block_size=w.block_size)



# ---- scores for the budgeted eviction selection -----------------------------------------------
#
# Eviction ranks (layer, KV head, position) entries by an attention score. The scores are drawn
# directly (nothing here computes attention): "lognormal" draws exp(sigma * z), z ~ N(0, 1), a
# positive, heavy-tailed spread over orders of magnitude with a few large "heavy hitters", the
# shape of accumulated attention mass; "levels" draws from a handful of values (heavy ties, so the
# (layer, head, position) tie-break decides many entries); "normal" draws z itself (signs and
# zeros mixed); "equal" gives every entry the same score (every entry ties).

EVICT_PRESETS = {
    # LLaMA-7B-shaped model (32 layers, 32 KV heads) at the 4096-token context of C2.
    "E1": dict(num_layers=32, num_heads=32, num_tokens=4096, budget_frac=0.25, kind="lognormal",
               sigma=2.0, seed=2001),
    # The long-context shape of C5 (8 KV heads, 131072 positions) over 32 layers.
    "E2": dict(num_layers=32, num_heads=8, num_tokens=131072, budget_frac=0.10, kind="lognormal",
               sigma=2.0, seed=2002),
}


def make_scores(num_layers: int, num_heads: int, num_tokens: int, kind: str = "lognormal",
                seed: int = 0, device="cpu", sigma: float = 2.0, row_stride: Optional[int] = None,
                levels=(0.0, 0.25, 0.5, 1.0)) -> torch.Tensor:
    """Seeded fp32 scores [L, H, N] (a view with rows ``row_stride`` apart when given)."""
    stride = num_tokens if row_stride is None else int(row_stride)
    if stride < num_tokens:
        raise ValueError("row_stride < num_tokens")
    rows = num_layers * num_heads
    store = torch.empty((rows, stride), dtype=torch.float32, device=device)
    gen = _generator(seed, 6, device)
    if kind in ("lognormal", "normal"):
        _fill_normal(store, gen, 1.0)
        if kind == "lognormal":
            store.mul_(sigma).exp_()
    elif kind == "levels":
        idx = torch.randint(0, len(levels), (rows, stride), generator=gen, device=device)
        store.copy_(torch.tensor(list(levels), dtype=torch.float32, device=device)[idx])
    elif kind == "equal":
        store.fill_(1.0)
    else:
        raise ValueError(f"unknown score kind {kind!r}")
    if stride > num_tokens:
        store[:, num_tokens:] = float("nan")  # never read
    return store[:, :num_tokens].view(num_layers, num_heads, num_tokens) if stride == num_tokens \
        else store.view(num_layers, num_heads, stride)[:, :, :num_tokens]
