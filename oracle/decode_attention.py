"""Plain fp64 definition of single-token decode attention over a (paged) KV cache.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): used only by tests, the smoke check and the
CPU-baseline leg of the bench. No product code imports it.

Sources, by page title and section:

* Ch. 19 "Inference Systems and Performance Engineering" (第19章 推理系统与性能工程)
  - §19.4.1: decode step t attends with softmax(Q_t Kᵀ/√d)·V over every cached position.
  - §19.6.1: the standard, unfused form materialises the score row, takes its softmax, then
    forms the weighted sum of V.
  - §19.6.2: the numerically stable softmax subtracts the row maximum before exponentiating.
  - §19.7.3: PagedAttention keeps the KV cache in fixed-size blocks reached through a
    per-sequence block table (logical block -> physical block).
* Ch. 10 "System Model of Throughput and Latency" (第十章 吞吐与延迟的系统模型)
  - §4: under GQA several query heads share one KV head; the unique-KV traffic model assumes
    the shared KV is read once.

Readings taken where the pages leave a point open:

* GQA grouping: query head ``h`` reads KV head ``h // g`` with ``g = h_q // h_kv``.
* ``d`` in 1/√d is the per-head dimension; a caller-given scale overrides it.
* ``ctx_lens[b]`` counts every position to attend, the current token included (the cache was
  appended before the step); there is no mask inside those positions.
* ``ctx_lens[b] == 0`` yields a zero output row (softmax of an empty set is undefined).
* Window / sinks (Ch. 19 §19.4.3 describes keeping only the last W tokens, and StreamingLLM's
  first "sink" tokens plus a recent window): with a window W the attended positions are the
  first ``num_sinks`` positions and the last W positions of the sequence, each once.
* Cache arrays are indexed ``[block, slot, kv_head, dim]``. Contiguous caches are the case with
  no block table: sequence ``b`` is block ``b`` and logical position ``t`` is slot ``t``.
* Storage types: ``float32`` arrays hold fp32 values; ``uint16`` arrays hold bf16 bit patterns.
  Both widen to fp64 exactly. All arithmetic is fp64; the single rounding to the fp32 output
  happens in :func:`round_to_f32` (round to nearest even).
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "widen",
    "logical_rows",
    "attended_positions",
    "stable_softmax",
    "attend_one",
    "decode_attention",
    "round_to_f32",
]


def widen(x: np.ndarray) -> np.ndarray:
    """Exact widening of stored values to fp64.

    ``uint16`` is read as bf16 bit patterns: the 16 bits become the high half of an fp32 word,
    which is then converted to fp64. Both steps are exact. ``float32``/``float64`` convert
    exactly as well.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported storage dtype {x.dtype} (expected float32 or bf16 bits as uint16)")


def logical_rows(cache: np.ndarray, block_table, b: int, kv_head: int, length: int,
                 block_size: int | None) -> np.ndarray:
    """Rows of logical positions ``0 .. length-1`` of sequence ``b`` for one KV head, in fp64.

    Block-table translation of Ch. 19 §19.7.3: logical position ``t`` lives in physical block
    ``block_table[b][t // block_size]`` at slot ``t % block_size``. Without a block table the
    cache is contiguous per sequence (block ``b``, slot ``t``).

    ``cache`` is indexed ``[block, slot, kv_head, dim]``; the result has shape ``[length, dim]``.
    """
    t = np.arange(length, dtype=np.int64)
    if block_table is None:
        blk = np.full(length, b, dtype=np.int64)
        slot = t
    else:
        if block_size is None:
            raise ValueError("a paged cache needs block_size")
        bt = np.asarray(block_table)
        blk = bt[b, t // block_size].astype(np.int64)
        slot = t % block_size
    return widen(cache[blk, slot, kv_head, :])


def stable_softmax(x: np.ndarray) -> np.ndarray:
    """softmax with the row maximum subtracted first (Ch. 19 §19.6.2)."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x)
    e = np.exp(x - m)
    return e / np.sum(e)


def attend_one(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """One query row against its cached rows, in the standard unfused order of Ch. 19 §19.6.1.

    S = scale · K q (the whole score row is materialised), P = softmax(S), o = P V.
    ``q``: [d]; ``keys``/``values``: [T, d]; returns [d] in fp64.
    """
    scores = scale * (keys @ q)
    probs = stable_softmax(scores)
    return probs @ values


def attended_positions(length: int, window: int | None = None, num_sinks: int = 0) -> np.ndarray:
    """Positions a decode step attends to among ``0 .. length-1``.

    Without a window: all of them. With a window W (Ch. 19 §19.4.3: a sliding window keeps the
    last W tokens; StreamingLLM additionally keeps the first tokens, the attention sinks): the
    first ``num_sinks`` positions and the last W positions, each position once.
    """
    t = np.arange(length, dtype=np.int64)
    if window is None:
        return t
    return t[(t < num_sinks) | (t >= length - window)]


def decode_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, ctx_lens,
                     block_table=None, *, block_size: int | None = None,
                     scale: float | None = None, window: int | None = None,
                     num_sinks: int = 0) -> np.ndarray:
    """Decode attention for a batch of sequences, one new query token per sequence.

    Parameters
    ----------
    q : [B, h_q, d] float32 values or bf16 bits (uint16).
    k_cache, v_cache : [num_blocks, block_slots, h_kv, d], same storage conventions. For a
        contiguous cache pass ``block_table=None`` (block ``b`` is sequence ``b``).
    ctx_lens : [B] integers, positions attended per sequence (current token included).
    block_table : [B, max_blocks] integers or ``None``.
    block_size : tokens per block for a paged cache.
    scale : score scale; ``None`` means 1/√d (Ch. 19 §19.4.1).
    window, num_sinks : restrict attention to :func:`attended_positions` (``None``: all).

    Returns
    -------
    [B, h_q, d] fp64 outputs; rows with ``ctx_lens[b] == 0`` are zero.
    """
    q = np.asarray(q)
    batch, h_q, d = q.shape
    h_kv = k_cache.shape[2]
    if k_cache.shape[3] != d or v_cache.shape[3] != d or v_cache.shape[2] != h_kv:
        raise ValueError("q, k_cache and v_cache disagree on head count or head dimension")
    if h_q % h_kv != 0:
        raise ValueError("h_q must be a multiple of h_kv")
    group = h_q // h_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qf = widen(q)
    ctx = np.asarray(ctx_lens).astype(np.int64)
    out = np.zeros((batch, h_q, d), dtype=np.float64)
    for b in range(batch):
        length = int(ctx[b])
        if length <= 0:
            continue
        keep = attended_positions(length, window, num_sinks)
        for kvh in range(h_kv):
            keys = logical_rows(k_cache, block_table, b, kvh, length, block_size)[keep]
            values = logical_rows(v_cache, block_table, b, kvh, length, block_size)[keep]
            for j in range(group):
                h = kvh * group + j
                out[b, h] = attend_one(qf[b, h], keys, values, scale)
    return out


def round_to_f32(x: np.ndarray) -> np.ndarray:
    """The single rounding of the fp64 result to the fp32 output (round to nearest even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)
