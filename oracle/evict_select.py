"""Plain reference for budgeted KV eviction selection.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Source: Ch. 19 "Inference Systems and Performance Engineering" (第19章 推理系统与性能工程)
§19.4.3 (KV-cache compression; the programming exercise on eviction). Given an attention score
for every (layer l, head h, token t) and a global budget of M kept KV entries, the page's rule is:

1. the current position C of every (layer, head) is kept unconditionally: L·H slots, leaving
   M − L·H for the rest;
2. every other (l, h, t) competes in one global pool, whatever its layer or head (so different
   layers may keep different numbers of tokens);
3. the pool is ordered by the key (−score, l, h, t) ascending: higher score first, ties broken by
   layer, then head, then token, each ascending;
4. the key is a total order, so the kept set is unique.

The page contrasts a naive selection (repeatedly scanning the table for the best remaining entry)
with a single global sort; the oracle is the global sort: one library sort of the pool by that
key, the first M − L·H entries kept.

Readings taken where the page is silent:

* Scores are real numbers compared as values (so −0.0 and +0.0 tie and fall to the index
  tie-break); ±inf are allowed; NaN has no place in the order and is rejected.
* C is one position index shared by all (layer, head) rows (the token being generated);
  it defaults to the last position N − 1.
* M < L·H still keeps every current position (rule 1 is unconditional) and nothing else;
  M − L·H at or above the pool size keeps everything.
"""

from __future__ import annotations

import numpy as np

__all__ = ["evict_select"]


def evict_select(scores, budget: int, current: int | None = None) -> np.ndarray:
    """Kept-entry mask of the budgeted selection.

    scores : [L, H, N] real array (any float dtype; compared exactly after widening to fp64,
             which is exact for fp32 and bf16 values).
    budget : M, the total number of kept (l, h, t) entries.
    current: C, the current position kept in every (l, h) row (default N − 1).
    Returns a bool array [L, H, N], True where the entry is kept.
    """
    s = np.asarray(scores, dtype=np.float64)
    if s.ndim != 3:
        raise ValueError("scores must be [L, H, N]")
    L, H, N = s.shape
    if N < 1:
        raise ValueError("every (layer, head) row needs at least the current position")
    C = N - 1 if current is None else int(current)
    if not 0 <= C < N:
        raise ValueError("current position out of range")
    if np.isnan(s).any():
        raise ValueError("NaN scores have no place in the order")

    keep = np.zeros((L, H, N), dtype=bool)
    keep[:, :, C] = True                       # rule 1
    free = int(budget) - L * H
    if free <= 0:
        return keep

    # Rule 2: one pool of every (l, h, t) with t != C.
    l_idx, h_idx, t_idx = np.meshgrid(np.arange(L), np.arange(H), np.arange(N), indexing="ij")
    pool = t_idx != C
    neg = -s[pool]
    l_p, h_p, t_p = l_idx[pool], h_idx[pool], t_idx[pool]
    # Rule 3: ascending by (-score, l, h, t); numpy's lexsort takes the primary key last.
    # -(+0.0) and -(-0.0) compare equal, so signed zeros tie as values do.
    order = np.lexsort((t_p, h_p, l_p, neg))
    chosen = order[:free]
    keep[l_p[chosen], h_p[chosen], t_p[chosen]] = True
    return keep
