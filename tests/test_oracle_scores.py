"""Pins of the per-position attention-weight oracle ``oracle.position_scores`` (CPU only).

* every attending query head's weights sum to 1, so a sequence's scores per KV head sum to g;
* one position gets all of it (g); q = 0 spreads it evenly (g / T);
* two positions follow the logistic function of the score difference (pins scale and sign);
* for MHA the weights reproduce the already-pinned decode output: sum_t score_t v_t = out;
* positions outside the length or the window score exactly 0, and the weights of the attended
  ones equal a full-attention run over exactly those rows gathered by hand;
* paged and contiguous caches agree.
"""

import math

import numpy as np
import pytest

from oracle import decode_attention, position_scores


@pytest.fixture
def rng():
    return np.random.default_rng(17)


def test_scores_sum_to_the_group_size(rng):
    B, hkv, g, d, T = 3, 2, 4, 16, 40
    q = rng.standard_normal((B, hkv * g, d)).astype(np.float32)
    k = rng.standard_normal((B, T, hkv, d)).astype(np.float32)
    lens = [40, 7, 0]
    s = position_scores(q, k, lens)
    assert s.shape == (B, hkv, 40)
    np.testing.assert_allclose(s[0].sum(-1), g, rtol=1e-12)
    np.testing.assert_allclose(s[1].sum(-1), g, rtol=1e-12)
    assert (s[1, :, 7:] == 0).all() and (s[2] == 0).all()
    assert (s >= 0).all()


def test_single_position_and_zero_query():
    q = np.zeros((1, 4, 8), np.float32)
    k = np.random.default_rng(0).standard_normal((1, 5, 2, 8)).astype(np.float32)
    s = position_scores(q, k, [1])
    assert s.shape == (1, 2, 1) and (s == 2.0).all()
    s = position_scores(q, k, [5])
    np.testing.assert_allclose(s, np.full((1, 2, 5), 2.0 / 5), rtol=1e-14)


def test_two_positions_follow_the_logistic_function(rng):
    d = 8
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    k = rng.standard_normal((1, 2, 1, d)).astype(np.float32)
    s = position_scores(q, k, [2], scale=0.7)
    qd, kd = q.astype(np.float64)[0, 0], k.astype(np.float64)[0, :, 0]
    z = 0.7 * (kd[1] @ qd - kd[0] @ qd)
    assert math.isclose(s[0, 0, 0], 1.0 / (1.0 + math.exp(z)), rel_tol=1e-13)
    assert math.isclose(s[0, 0, 1], 1.0 / (1.0 + math.exp(-z)), rel_tol=1e-13)


def test_mha_weights_reproduce_the_decode_output(rng):
    B, h, d, T = 2, 3, 16, 30
    q = rng.standard_normal((B, h, d)).astype(np.float32)
    k = rng.standard_normal((B, T, h, d)).astype(np.float32)
    v = rng.standard_normal((B, T, h, d)).astype(np.float32)
    lens = [30, 11]
    s = position_scores(q, k, lens)
    out = decode_attention(q, k, v, lens)
    for b in range(B):
        for hh in range(h):
            got = s[b, hh, :lens[b]] @ v[b, :lens[b], hh].astype(np.float64)
            np.testing.assert_allclose(got, out[b, hh], rtol=1e-12, atol=1e-14)


def test_window_scores_only_the_kept_positions(rng):
    d, T, W, n = 8, 50, 10, 3
    q = rng.standard_normal((1, 2, d)).astype(np.float32)
    k = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    s = position_scores(q, k, [T], window=W, num_sinks=n)
    kept = list(range(n)) + list(range(T - W, T))
    others = [t for t in range(T) if t not in kept]
    assert (s[0, 0, others] == 0).all()
    ref = position_scores(q, k[:, kept], [len(kept)])
    np.testing.assert_allclose(s[0, 0, kept], ref[0, 0], rtol=1e-13)


def test_paged_equals_contiguous(rng):
    B, hkv, d, bs = 2, 2, 8, 4
    lens = [9, 6]
    q = rng.standard_normal((B, 2 * hkv, d)).astype(np.float32)
    k = rng.standard_normal((B, 12, hkv, d)).astype(np.float32)
    nblk = 3
    perm = rng.permutation(B * nblk)
    paged = np.zeros((B * nblk, bs, hkv, d), np.float32)
    table = np.zeros((B, nblk), np.int64)
    for b in range(B):
        for j in range(nblk):
            table[b, j] = perm[b * nblk + j]
            paged[table[b, j]] = k[b, j * bs:(j + 1) * bs]
    a = position_scores(q, k, lens)
    c = position_scores(q, paged, lens, table, block_size=bs)
    np.testing.assert_array_equal(a, c)
