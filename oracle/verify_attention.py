"""Plain fp64 reference for γ-query verification attention (speculative decoding's check step).

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Source: Ch. 19 "Inference Systems and Performance Engineering" (第19章 推理系统与性能工程)
§19.8 — a small draft model proposes γ tokens and the target model checks all γ positions in a
single forward pass (a γ×d-shaped product instead of γ sequential steps). The attention of that
pass is what is computed here; the acceptance rule that follows it needs the models' output
distributions and is not part of this path.

Readings taken where the page is silent:

* The γ proposed tokens have been appended to the cache before the check, so ``ctx_lens[b]``
  (T) counts them: they are positions T−γ .. T−1, and query j (0-based) is the token at
  position T−γ+j.
* Causality among the proposed tokens: query j attends to positions 0 .. T−γ+j, i.e. to the
  first T_j = T−γ+1+j positions, exactly as a single-token decode step over a sequence of
  length T_j would. T_j <= 0 gives a zero row (an empty softmax, as for an empty context).
* A window W and sinks apply per query: query j attends to ``attended_positions(T_j, W, n)``.
"""

from __future__ import annotations

import math

import numpy as np

from .decode_attention import attend_one, attended_positions, logical_rows, widen

__all__ = ["verify_attention"]


def verify_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, ctx_lens,
                     block_table=None, *, block_size: int | None = None,
                     scale: float | None = None, window: int | None = None,
                     num_sinks: int = 0) -> np.ndarray:
    """Attention of γ new query tokens per sequence, causal among themselves.

    q : [B, γ, h_q, d] (float32 values or bf16 bits as uint16); caches, block table, scale,
    window and sinks as for :func:`oracle.decode_attention.decode_attention`.
    Returns [B, γ, h_q, d] fp64.
    """
    q = np.asarray(q)
    batch, gamma, h_q, d = q.shape
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
    out = np.zeros((batch, gamma, h_q, d), dtype=np.float64)
    for b in range(batch):
        total = int(ctx[b])
        for j in range(gamma):
            length = total - (gamma - 1 - j)  # positions visible to the token at T-γ+j
            if length <= 0:
                continue
            keep = attended_positions(length, window, num_sinks)
            for kvh in range(h_kv):
                keys = logical_rows(k_cache, block_table, b, kvh, length, block_size)[keep]
                values = logical_rows(v_cache, block_table, b, kvh, length, block_size)[keep]
                for i in range(group):
                    h = kvh * group + i
                    out[b, j, h] = attend_one(qf[b, j, h], keys, values, scale)
    return out
