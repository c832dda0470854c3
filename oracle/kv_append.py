"""Plain reference for appending one token's K/V rows to a (paged) KV cache.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Sources: Ch. 10 "System Model of Throughput and Latency" (第十章 吞吐与延迟的系统模型) §4 —
every decode step writes the new token's key and value for every layer and KV head (the new-KV
write term of the traffic model) and the step reuses them right away; Ch. 19 "Inference
Systems and Performance Engineering" (第19章 推理系统与性能工程) §19.7.3 — the cache grows block by
block through the block table, so logical position t of sequence b lives in physical block
``block_table[b][t // block_size]`` at slot ``t % block_size``.

Reading: a negative position means "this sequence appends nothing this step" (an idle slot in a
batch); positions at or past the cache's capacity are not written either.
"""

from __future__ import annotations

import numpy as np

__all__ = ["append_kv"]


def append_kv(cache: np.ndarray, new_rows: np.ndarray, positions, block_table=None, *,
              block_size: int | None = None, capacity: int | None = None) -> np.ndarray:
    """Return a copy of ``cache`` with the new rows of every sequence stored.

    ``new_rows`` is ``[B, h_kv, dim]`` (one new token per sequence, stored at logical position
    ``positions[b]``) or ``[B, n, h_kv, dim]`` (n new tokens, token i stored at
    ``positions[b] + i``, e.g. the γ proposed tokens of a verification step), of the cache's
    dtype. ``cache`` is indexed ``[block, slot, kv_head, dim]`` (any storage dtype, copied bit
    for bit). Without a block table the cache is contiguous per sequence (block ``b``, slot =
    position) and ``capacity`` bounds the position; with one, ``block_table.shape[1] *
    block_size`` does. A negative first position skips the whole sequence; single tokens at or
    past the bound are skipped.
    """
    out = np.array(cache, copy=True)
    new_rows = np.asarray(new_rows)
    if new_rows.dtype != out.dtype:
        raise TypeError("new rows and cache must share a storage dtype")
    if new_rows.ndim == 3:
        new_rows = new_rows[:, None]
    if block_table is None:
        limit = capacity if capacity is not None else out.shape[1]
    else:
        bt = np.asarray(block_table)
        limit = bt.shape[1] * block_size
    for b, first in enumerate(np.asarray(positions).tolist()):
        first = int(first)
        if first < 0:
            continue
        for i in range(new_rows.shape[1]):
            pos = first + i
            if pos >= limit:
                continue
            if block_table is None:
                blk, slot = b, pos
            else:
                blk, slot = int(bt[b, pos // block_size]), pos % block_size
            out[blk, slot] = new_rows[b, i]
    return out
