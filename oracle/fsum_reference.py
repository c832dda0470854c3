"""Pure-Python second implementation of decode attention, for tiny shapes only.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

It restates the same plain definition as ``decode_attention.py`` (Ch. 19 "Inference Systems
and Performance Engineering", §19.4.1 operation, §19.6.1 unfused order, §19.6.2 max-subtracted
softmax, §19.7.3 block-table addressing) with Python floats, ``math.exp`` and the exactly
rounded ``math.fsum``, and without NumPy arithmetic. Agreement with the NumPy oracle pins the
oracle's indexing (GQA grouping, block translation, head/position axes) and its summations.
"""

from __future__ import annotations

import math
import struct

__all__ = ["decode_attention_fsum"]


def _value(raw, is_bf16: bool) -> float:
    """One stored element as a Python float (bf16 bits or an fp32 value)."""
    if is_bf16:
        return struct.unpack("<f", struct.pack("<I", (int(raw) & 0xFFFF) << 16))[0]
    return float(raw)


def decode_attention_fsum(q, k_cache, v_cache, ctx_lens, block_table=None, *,
                          block_size=None, scale=None, bf16=False, window=None, num_sinks=0):
    """Same contract as ``oracle.decode_attention.decode_attention`` (window and sinks included);
    returns nested lists.

    ``q`` is indexable as q[b][h][i]; caches as cache[block][slot][kv_head][i]. With
    ``bf16=True`` every stored element is a bf16 bit pattern.
    """
    batch = len(q)
    h_q = len(q[0])
    d = len(q[0][0])
    h_kv = len(k_cache[0][0])
    group = h_q // h_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = [[[0.0] * d for _ in range(h_q)] for _ in range(batch)]
    for b in range(batch):
        length = int(ctx_lens[b])
        if length <= 0:
            continue
        for h in range(h_q):
            kvh = h // group
            qv = [_value(q[b][h][i], bf16) for i in range(d)]
            rows = []
            for t in range(length):
                if window is not None and not (t < num_sinks or t >= length - window):
                    continue
                if block_table is None:
                    blk, slot = b, t
                else:
                    blk, slot = int(block_table[b][t // block_size]), t % block_size
                krow = [_value(k_cache[blk][slot][kvh][i], bf16) for i in range(d)]
                vrow = [_value(v_cache[blk][slot][kvh][i], bf16) for i in range(d)]
                rows.append((krow, vrow))
            scores = [scale * math.fsum(qv[i] * k[i] for i in range(d)) for k, _ in rows]
            m = max(scores)
            weights = [math.exp(s - m) for s in scores]
            total = math.fsum(weights)
            for i in range(d):
                out[b][h][i] = math.fsum(w * v[i] for w, (_, v) in zip(weights, rows)) / total
    return out
