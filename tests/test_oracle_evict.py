"""Pins of the eviction-selection oracle (CPU only).

``oracle.evict_select`` is the page's global sort (Ch. 19 §19.4.3 exercise). It is pinned by:

* a case worked by hand from the four rules (tests/golden/evict_worked_example.json), where every
  tie-break level and the exclusion of the current position decide an entry;
* the naive method the page contrasts with the sort (repeatedly scan the whole table for the
  best remaining entry), written here independently, on many tiny inputs with heavy ties,
  signed zeros and infinities;
* properties that hold at any size: the kept count, the threshold property of the key order,
  monotonicity in the budget, and the edge cases of the budget.

Planted mistakes (a tie-break in the wrong order, the current position left in the pool, ties
broken by token first) are shown to fail the pins.
"""

import json
import math
import os
import random

import numpy as np
import pytest

from oracle import evict_select

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "evict_worked_example.json")


def _naive(scores, budget, current):
    """The naive method: M - L*H rounds, each scanning the table in (l, h, t) order for the
    largest score not yet taken (strictly larger replaces, so the first in order wins ties)."""
    L, H, N = len(scores), len(scores[0]), len(scores[0][0])
    kept = {(l, h, current) for l in range(L) for h in range(H)}
    for _ in range(budget - L * H):
        best = None
        for l in range(L):
            for h in range(H):
                for t in range(N):
                    if (l, h, t) in kept:
                        continue
                    if best is None or scores[l][h][t] > scores[best[0]][best[1]][best[2]]:
                        best = (l, h, t)
        if best is None:
            break
        kept.add(best)
    return kept


def _as_set(mask):
    return {tuple(int(x) for x in idx) for idx in np.argwhere(mask)}


def test_worked_example():
    g = json.load(open(GOLDEN))
    assert g["source"]
    scores = np.array(g["scores"], dtype=np.float32)
    assert scores.shape == (g["L"], g["H"], g["N"])
    keep = evict_select(scores, g["budget"], g["current"])
    assert _as_set(keep) == {tuple(k) for k in g["kept"]}
    per_layer = keep.sum(axis=(1, 2))
    assert per_layer.tolist() == [6, 4]


def test_worked_example_catches_planted_mistakes():
    g = json.load(open(GOLDEN))
    scores = np.array(g["scores"], dtype=np.float64)
    want = {tuple(k) for k in g["kept"]}
    L, H, N, C, M = g["L"], g["H"], g["N"], g["current"], g["budget"]
    cands = [(l, h, t) for l in range(L) for h in range(H) for t in range(N) if t != C]
    currents = {(l, h, C) for l in range(L) for h in range(H)}

    def pick(keyfn, pool=cands, free=M - L * H):
        return currents | set(sorted(pool, key=keyfn)[:free])

    # the correct key reproduces the worked example ...
    assert pick(lambda e: (-scores[e], e[0], e[1], e[2])) == want
    # ... and each plausible slip does not
    assert pick(lambda e: (-scores[e], e[1], e[0], e[2])) != want        # head before layer
    assert pick(lambda e: (-scores[e], e[2], e[0], e[1])) != want        # token first
    assert pick(lambda e: (-scores[e], -e[0], e[1], e[2])) != want       # layer descending
    all_entries = cands + sorted(currents)
    assert pick(lambda e: (-scores[e], *e), pool=all_entries) != want     # current left in pool


def _tiny_cases(n, seed=3):
    rnd = random.Random(seed)
    levels = [0.0, -0.0, 0.25, 0.5, 1.0, -1.0, math.inf, -math.inf, 3.0]
    for _ in range(n):
        L, H, N = rnd.randint(1, 3), rnd.randint(1, 3), rnd.randint(1, 5)
        if rnd.random() < 0.5:
            vals = [[[rnd.choice(levels) for _ in range(N)] for _ in range(H)] for _ in range(L)]
        else:
            vals = [[[rnd.uniform(-2, 2) for _ in range(N)] for _ in range(H)] for _ in range(L)]
        C = rnd.randrange(N)
        M = rnd.randint(0, L * H * N + 2)
        yield vals, M, C


def test_matches_the_naive_method_on_tiny_inputs():
    for vals, M, C in _tiny_cases(400):
        keep = evict_select(np.array(vals, dtype=np.float32), M, C)
        want = _naive(np.array(vals, dtype=np.float32).astype(np.float64).tolist(), M, C)
        assert _as_set(keep) == want, (vals, M, C)


def test_kept_count_and_threshold_property():
    rng = np.random.default_rng(5)
    for _ in range(30):
        L, H, N = rng.integers(1, 5, size=3)
        s = rng.choice(np.array([0.0, 0.1, 0.2, 0.3], dtype=np.float32), size=(L, H, N))
        C = int(rng.integers(0, N))
        M = int(rng.integers(0, L * H * N + 3))
        keep = evict_select(s, M, C)
        pool = L * H * (N - 1)
        assert keep.sum() == L * H + min(max(M - L * H, 0), pool)
        assert keep[:, :, C].all()
        kept_keys = [(-float(s[l, h, t]), l, h, t) for l, h, t in np.argwhere(keep) if t != C]
        dropped = [(-float(s[l, h, t]), l, h, t) for l, h, t in np.argwhere(~keep)]
        if kept_keys and dropped:
            assert max(kept_keys) < min(dropped)


def test_monotone_in_the_budget():
    rng = np.random.default_rng(9)
    s = rng.standard_normal((3, 2, 7)).astype(np.float32)
    s[0, 0, :3] = 0.5  # some ties
    prev = evict_select(s, 0, 6)
    for M in range(1, 3 * 2 * 7 + 2):
        cur = evict_select(s, M, 6)
        assert (cur | prev).sum() == cur.sum()          # prev is a subset of cur
        assert cur.sum() - prev.sum() == (1 if 3 * 2 <= M <= 3 * 2 * 7 and M > 6 else 0)
        prev = cur


def test_budget_edges():
    s = np.arange(2 * 3 * 4, dtype=np.float32).reshape(2, 3, 4)
    only_current = np.zeros_like(s, dtype=bool)
    only_current[:, :, 1] = True
    for M in (0, 1, 5, 6):  # at or below L*H: only the current positions
        assert np.array_equal(evict_select(s, M, 1), only_current)
    assert evict_select(s, 24, 1).all()
    assert evict_select(s, 10**9, 1).all()
    # N == 1: the current position is the whole row
    assert evict_select(np.ones((2, 2, 1), np.float32), 100).all()


def test_signed_zeros_tie_and_fall_to_the_index_order():
    s = np.array([[[-0.0, 0.0, -0.0, 1.0]]], dtype=np.float32)
    keep = evict_select(s, 3, 3)  # two free slots among three equal zeros
    assert keep[0, 0].tolist() == [True, True, False, True]
    s2 = np.array([[[0.0, -0.0, 0.0, 1.0]]], dtype=np.float32)
    assert evict_select(s2, 3, 3)[0, 0].tolist() == [True, True, False, True]


def test_infinities_order_and_nan_is_rejected():
    s = np.array([[[-math.inf, 1e30, math.inf, 0.0, 5.0]]], dtype=np.float32)
    assert evict_select(s, 3, 4)[0, 0].tolist() == [False, True, True, False, True]
    with pytest.raises(ValueError):
        evict_select(np.array([[[0.0, float("nan"), 1.0]]]), 2)


def test_current_defaults_to_the_last_position_and_is_validated():
    s = np.zeros((1, 1, 4), np.float32)
    assert evict_select(s, 1)[0, 0].tolist() == [False, False, False, True]
    with pytest.raises(ValueError):
        evict_select(s, 1, 4)
    with pytest.raises(ValueError):
        evict_select(np.zeros((2, 3)), 1)
