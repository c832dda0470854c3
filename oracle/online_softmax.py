"""Blockwise online-softmax recurrence and merge of running states, in fp64.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Source: Ch. 19 "Inference Systems and Performance Engineering" (第19章 推理系统与性能工程),
§19.6.2 (online softmax recurrence), §19.6.3 (tiled forward pass: state initialised to
m = -inf, l = 0, O = 0, each block updates it, the result is O / l), and self-test question Q4
of the same chapter, which restates the recurrence.

The running state after some blocks is the triple (m, l, O):

* m — the maximum score seen so far;
* l — the sum of exp(x_j - m) over the positions seen so far;
* O — the unnormalised sum of exp(x_j - m) · v_j over the positions seen so far.

A new block with maximum m~ updates it as: m' = max(m, m~); c = exp(m - m'); l' = c·l + the
block's sum of exp(x_j - m'); O' = c·O + the block's sum of exp(x_j - m')·v_j. The chapter
argues this is exact (only e^(a+b) = e^a·e^b is used), so O/l equals the full softmax-weighted
sum up to rounding order.

Reading for the empty state (pages: c is said to lie in (0, 1], yet m starts at -inf, which
makes the first c equal to 0): c lies in [0, 1]; a state with m = -inf and l = 0 is the
identity of :func:`merge_states`, which skips it so that (-inf) - (-inf) never occurs.

:func:`merge_states` combines two states built over disjoint position sets. It is the same
rescale-and-add step with a whole second state in place of one raw block; it is what a
split-KV decode merges per split.
"""

from __future__ import annotations

import itertools
import math
from typing import Iterable, Sequence

import numpy as np

__all__ = [
    "EMPTY_STATE",
    "block_state",
    "online_softmax",
    "merge_states",
    "merge_many",
    "finalize_state",
    "compositions",
]

NEG_INF = -math.inf


def EMPTY_STATE(d: int):
    """The state before any block (§19.6.3): m = -inf, l = 0, O = 0."""
    return (NEG_INF, 0.0, np.zeros(d, dtype=np.float64))


def block_state(scores: np.ndarray, values: np.ndarray):
    """The state of one block on its own: (max, sum of exp(x - max), sum of exp(x - max)·v)."""
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if scores.size == 0:
        return EMPTY_STATE(values.shape[1])
    m = float(np.max(scores))
    e = np.exp(scores - m)
    return (m, float(np.sum(e)), e @ values)


def online_softmax(scores: np.ndarray, values: np.ndarray, blocks: Iterable[Sequence[int]]):
    """Run the recurrence of §19.6.2 over ``blocks`` (index lists) of one score row.

    Returns ``(o, state, trace)`` where ``o = O/l`` is the attention output, ``state`` the
    final (m, l, O), and ``trace`` a list of (m_k, c) per block, for checking that m never
    decreases and c never exceeds 1.
    """
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    m, l, o_acc = EMPTY_STATE(values.shape[1])
    trace = []
    for idx in blocks:
        idx = np.asarray(idx, dtype=np.int64)
        x = scores[idx]
        m_tilde = float(np.max(x))
        m_next = max(m, m_tilde)
        c = math.exp(m - m_next)  # exp(-inf) == 0 on the first block
        e = np.exp(x - m_next)
        l = c * l + float(np.sum(e))
        o_acc = c * o_acc + e @ values[idx]
        m = m_next
        trace.append((m, c))
    return finalize_state((m, l, o_acc)), (m, l, o_acc), trace


def merge_states(a, b):
    """Combine two running states over disjoint position sets.

    M = max(m_a, m_b); l = e^(m_a-M)·l_a + e^(m_b-M)·l_b; O likewise. An empty operand
    (m = -inf) is returned unchanged as the identity.
    """
    m_a, l_a, o_a = a
    m_b, l_b, o_b = b
    if m_a == NEG_INF:
        return (m_b, l_b, np.array(o_b, dtype=np.float64))
    if m_b == NEG_INF:
        return (m_a, l_a, np.array(o_a, dtype=np.float64))
    m = max(m_a, m_b)
    w_a = math.exp(m_a - m)
    w_b = math.exp(m_b - m)
    return (m, w_a * l_a + w_b * l_b, w_a * np.asarray(o_a) + w_b * np.asarray(o_b))


def merge_many(states, d: int):
    """Left fold of :func:`merge_states` over ``states``, starting from the empty state."""
    acc = EMPTY_STATE(d)
    for s in states:
        acc = merge_states(acc, s)
    return acc


def finalize_state(state) -> np.ndarray:
    """O / l; an empty state (l == 0) gives the zero vector (the empty-context reading)."""
    m, l, o_acc = state
    o_acc = np.asarray(o_acc, dtype=np.float64)
    if l == 0.0:
        return np.zeros_like(o_acc)
    return o_acc / l


def compositions(n: int):
    """Every split of positions 0..n-1 into consecutive non-empty blocks (2^(n-1) of them)."""
    for cuts in itertools.product((False, True), repeat=max(n - 1, 0)):
        blocks, start = [], 0
        for i, cut in enumerate(cuts, start=1):
            if cut:
                blocks.append(list(range(start, i)))
                start = i
        blocks.append(list(range(start, n)))
        yield blocks
