"""Plain fp64 reference for the attention weight each cached position receives in a decode step.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Source: Ch. 19 "Inference Systems and Performance Engineering" (第19章 推理系统与性能工程)
§19.4.3 — eviction policies rank cached tokens by the attention they receive (H2O's observation:
a few "heavy hitter" tokens collect most of the attention mass), and the eviction exercise takes
one score per (layer, head, token). The weights themselves are the softmax of §19.4.1 / §19.6.2:
P = softmax(scale · K q) over the attended positions.

Readings taken where the page is silent:

* The unit that is kept or evicted is a KV head's entry, so the score of (sequence b, KV head
  kvh, position t) is the sum over the g query heads that share that KV head of the weight each
  gives position t (their weights each sum to 1, so a sequence's scores per KV head sum to g).
* Positions a step does not attend (past ctx_lens[b], or outside a window) score 0.
* Accumulating scores across decode steps (H2O's running sum) is the caller's addition of
  successive results.
"""

from __future__ import annotations

import math

import numpy as np

from .decode_attention import attended_positions, logical_rows, stable_softmax, widen

__all__ = ["position_scores"]


def position_scores(q: np.ndarray, k_cache: np.ndarray, ctx_lens, block_table=None, *,
                    block_size: int | None = None, scale: float | None = None,
                    window: int | None = None, num_sinks: int = 0,
                    max_len: int | None = None) -> np.ndarray:
    """Attention weight per (sequence, KV head, position), summed over the KV head's query heads.

    q : [B, h_q, d] (float32 values or bf16 bits as uint16); k_cache [blocks, slots, h_kv, d];
    block table, scale, window and sinks as for :func:`oracle.decode_attention.decode_attention`.
    Returns [B, h_kv, max_len] fp64 (max_len defaults to max(ctx_lens)).
    """
    q = np.asarray(q)
    batch, h_q, d = q.shape
    h_kv = k_cache.shape[2]
    if k_cache.shape[3] != d:
        raise ValueError("q and k_cache disagree on the head dimension")
    if h_q % h_kv != 0:
        raise ValueError("h_q must be a multiple of h_kv")
    group = h_q // h_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ctx = np.asarray(ctx_lens).astype(np.int64)
    width = int(ctx.max()) if max_len is None and ctx.size else int(max_len or 0)
    qf = widen(q)
    out = np.zeros((batch, h_kv, width), dtype=np.float64)
    for b in range(batch):
        length = int(ctx[b])
        if length <= 0:
            continue
        keep = attended_positions(length, window, num_sinks)
        for kvh in range(h_kv):
            keys = logical_rows(k_cache, block_table, b, kvh, length, block_size)[keep]
            for j in range(group):
                weights = stable_softmax(scale * (keys @ qf[b, kvh * group + j]))
                out[b, kvh, keep] += weights
    return out
