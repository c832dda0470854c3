"""Brute-force pins of the online-softmax recurrence and of the state merge (CPU only).

Ch. 19 "Inference Systems and Performance Engineering", §19.6.2 argues that the blockwise
recurrence on (m, l, O) is exact: it equals the full max-subtracted softmax up to rounding
order, m never decreases and the rescale factor c never exceeds 1. These tests check that
claim over every split of short rows into consecutive blocks, and check that merging split
states (what a split-KV decode does) is associative and commutative with the empty state as its
identity. Two planted mistakes (a dropped rescale, a merge that forgets one side's weight) must
be caught.
"""

import itertools
import math

import numpy as np
import pytest

from oracle import (EMPTY_STATE, attend_one, block_state, finalize_state, merge_many,
                    merge_states, online_softmax)
from oracle.online_softmax import compositions


def _row(rng, T, d, spread=3.0):
    scores = rng.standard_normal(T) * spread
    values = rng.standard_normal((T, d))
    return scores, values


def _full(scores, values):
    # attend_one with K = scores as a 1-wide key matrix and q = [1]: softmax(scores) @ values
    return attend_one(np.array([1.0]), scores[:, None], values, 1.0)


def test_compositions_enumerates_all_splits():
    for n in range(1, 8):
        comps = list(compositions(n))
        assert len(comps) == 2 ** (n - 1)
        assert len({tuple(map(tuple, c)) for c in comps}) == len(comps)
        for c in comps:
            assert [i for blk in c for i in blk] == list(range(n))


@pytest.mark.parametrize("T", list(range(1, 11)))
def test_recurrence_equals_full_softmax_for_every_block_split(rng, T):
    scores, values = _row(rng, T, 5)
    full = _full(scores, values)
    for blocks in compositions(T):
        out, state, trace = online_softmax(scores, values, blocks)
        np.testing.assert_allclose(out, full, rtol=1e-12, atol=1e-14)
        ms = [m for m, _ in trace]
        cs = [c for _, c in trace]
        assert all(b >= a for a, b in zip(ms, ms[1:]))          # m is non-decreasing
        assert all(0.0 <= c <= 1.0 for c in cs)                 # c in [0, 1]
        assert cs[0] == 0.0                                     # first block: exp(-inf) = 0
        assert state[0] == np.max(scores)


def test_recurrence_survives_large_scores(rng):
    scores = np.array([800.0, 790.0, -5.0, 805.0, 0.0])
    values = rng.standard_normal((5, 3))
    out, _, _ = online_softmax(scores, values, [[0, 1], [2], [3, 4]])
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out, _full(scores, values), rtol=1e-12)


def test_dropping_the_rescale_is_detected(rng):
    """Planted mistake: without c the states mix different reference maxima."""
    scores, values = _row(rng, 6, 4)
    scores[4] = 6.0  # a later block raises the maximum
    blocks = [[0, 1, 2], [3, 4, 5]]
    m, l, o = EMPTY_STATE(4)
    for idx in blocks:
        x = scores[idx]
        m = max(m, float(np.max(x)))
        e = np.exp(x - m)
        l = l + e.sum()                    # c omitted
        o = o + e @ values[idx]            # c omitted
    wrong = o / l
    assert np.max(np.abs(wrong - _full(scores, values))) > 1e-3


def _states_for(scores, values, blocks):
    return [block_state(scores[np.asarray(b)], values[np.asarray(b)]) for b in blocks]


@pytest.mark.parametrize("T", [4, 7, 10])
def test_merge_is_associative_and_commutative(rng, T):
    scores, values = _row(rng, T, 3)
    full = _full(scores, values)
    for blocks in compositions(T):
        if len(blocks) > 4:
            continue
        states = _states_for(scores, values, blocks)
        for order in itertools.permutations(range(len(states))):
            ordered = [states[i] for i in order]
            left = merge_many(ordered, 3)
            np.testing.assert_allclose(finalize_state(left), full, rtol=1e-12, atol=1e-14)
            # right fold
            acc = EMPTY_STATE(3)
            for s in reversed(ordered):
                acc = merge_states(s, acc)
            np.testing.assert_allclose(finalize_state(acc), full, rtol=1e-12, atol=1e-14)


def test_merge_of_non_consecutive_position_sets(rng):
    """Splits need not be contiguous runs: any partition of positions merges to the same row."""
    scores, values = _row(rng, 9, 4)
    parts = [[0, 4, 8], [1, 2], [3, 5, 6, 7]]
    merged = merge_many(_states_for(scores, values, parts), 4)
    np.testing.assert_allclose(finalize_state(merged), _full(scores, values), rtol=1e-12)


def test_empty_state_is_the_merge_identity(rng):
    scores, values = _row(rng, 5, 3)
    s = block_state(scores, values)
    e = EMPTY_STATE(3)
    for merged in (merge_states(s, e), merge_states(e, s)):
        assert merged[0] == s[0] and merged[1] == s[1]
        assert np.array_equal(merged[2], s[2])
    both_empty = merge_states(e, e)
    assert both_empty[0] == -math.inf and both_empty[1] == 0.0
    assert np.all(finalize_state(both_empty) == 0.0)


def test_forgetting_one_weight_in_the_merge_is_detected(rng):
    """Planted mistake: adding O_b without e^(m_b - M) breaks the merge."""
    scores, values = _row(rng, 8, 3)
    scores[:4] += 5.0  # the first half holds the maximum, so b's weight is < 1
    a = block_state(scores[:4], values[:4])
    b = block_state(scores[4:], values[4:])
    m = max(a[0], b[0])
    wa = math.exp(a[0] - m)
    wrong = (wa * a[2] + b[2]) / (wa * a[1] + b[1])
    good = finalize_state(merge_states(a, b))
    np.testing.assert_allclose(good, _full(scores, values), rtol=1e-12)
    assert a[0] > b[0]
    assert np.max(np.abs(wrong - good)) > 1e-3
