"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

The pages print no numeric attention output, so the oracle is pinned by closed forms,
invariants, special cases that reduce to textbook routines, and an independent pure-Python
implementation. Each pin is chosen so that a plausible slip fails it:

* a wrong V row / head index or block translation   -> T=1, GQA, paged and fsum pins
* a wrong scale (1/d instead of 1/sqrt(d)) or sign   -> logistic closed form, scale pin
* missing normalisation or a dropped term            -> mean, identical-rows, fsum pins
* K and V paired from different positions            -> logistic and dominant-key pins
"""

import math

import numpy as np
import pytest

from oracle import decode_attention, stable_softmax, widen, round_to_f32, decode_attention_fsum


def _contig(rng, B, hkv, T, d, dtype=np.float32):
    """Random contiguous caches [B, T, hkv, d] (block b = sequence b)."""
    k = rng.standard_normal((B, T, hkv, d)).astype(dtype)
    v = rng.standard_normal((B, T, hkv, d)).astype(dtype)
    return k, v


def _to_bf16_bits(x):
    """Truncate fp32 values to bf16 bit patterns (any bf16 value is a valid test input)."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------------------------
# storage widening


def test_bf16_widening_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x4049],
                    dtype=np.uint16)
    got = widen(bits)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 0.0, -0.0, math.inf, -math.inf, 2.0 ** -133,
            3.140625]
    assert got.dtype == np.float64
    for g, w in zip(got, want):
        assert g == w
    assert math.copysign(1.0, got[4]) == -1.0
    assert np.isnan(widen(np.array([0x7FC0], dtype=np.uint16)))[0]


def test_fp32_widening_is_exact():
    x = np.array([1.0 + 2.0 ** -23, -3.0e-38, 1.0e38, 2.0 ** -149], dtype=np.float32)
    assert np.array_equal(widen(x), x.astype(np.float64))


# ---------------------------------------------------------------------------------------------
# softmax helper (Ch. 19 §19.6.2)


def test_stable_softmax_matches_unshifted_form_and_is_shift_invariant(rng):
    x = rng.standard_normal(50) * 3
    direct = np.exp(x) / np.exp(x).sum()  # the unshifted textbook form, fine at this range
    assert np.allclose(stable_softmax(x), direct, rtol=1e-14, atol=0)
    assert np.allclose(stable_softmax(x + 700.0), stable_softmax(x), rtol=1e-12, atol=0)
    assert abs(stable_softmax(x).sum() - 1.0) < 1e-15
    huge = np.array([1000.0, 999.0, -1000.0])
    p = stable_softmax(huge)
    assert np.all(np.isfinite(p)) and abs(p[0] / p[1] - math.e) < 1e-12


# ---------------------------------------------------------------------------------------------
# closed forms and special cases of the whole definition


@pytest.mark.parametrize("d", [8, 64, 128])
def test_single_position_returns_its_value_row_exactly(rng, d):
    k, v = _contig(rng, 2, 3, 1, d)
    q = rng.standard_normal((2, 6, d)).astype(np.float32)
    out = decode_attention(q, k, v, [1, 1])
    for b in range(2):
        for h in range(6):
            assert np.array_equal(out[b, h], v[b, 0, h // 2].astype(np.float64))


def test_identical_value_rows_return_that_row(rng):
    B, hkv, T, d = 2, 2, 37, 16
    k, _ = _contig(rng, B, hkv, T, d)
    row = rng.standard_normal((B, 1, hkv, d))
    v = np.broadcast_to(row, (B, T, hkv, d)).astype(np.float32)
    q = (rng.standard_normal((B, 4, d)) * 2).astype(np.float32)
    out = decode_attention(q, k, v, [T, T])
    for b in range(B):
        for h in range(4):
            np.testing.assert_allclose(out[b, h], v[b, 0, h // 2], rtol=1e-12, atol=1e-14)


def test_zero_query_gives_the_arithmetic_mean_of_values(rng):
    B, hkv, T, d = 1, 2, 53, 32
    k, v = _contig(rng, B, hkv, T, d)
    q = np.zeros((B, 2, d), dtype=np.float32)
    out = decode_attention(q, k, v, [T])
    for h in range(2):
        np.testing.assert_allclose(out[0, h], np.mean(v[0, :, h].astype(np.float64), axis=0),
                                   rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("d", [4, 64])
def test_two_positions_follow_the_logistic_closed_form(d):
    """q = a·e_i, k_0 = alpha·e_i, k_1 = 0: s_0 = a·alpha/sqrt(d), s_1 = 0, so the weight of
    position 0 is the logistic 1 / (1 + e^(-s_0)). Values are e_0 and e_1 (d >= 2)."""
    a, alpha, i = 1.5, 2.0, 1
    q = np.zeros((1, 1, d), dtype=np.float32)
    q[0, 0, i] = a
    k = np.zeros((1, 2, 1, d), dtype=np.float32)
    k[0, 0, 0, i] = alpha
    v = np.zeros((1, 2, 1, d), dtype=np.float32)
    v[0, 0, 0, 0] = 1.0
    v[0, 1, 0, 1] = 1.0
    out = decode_attention(q, k, v, [2])
    s0 = a * alpha / math.sqrt(d)
    w0 = 1.0 / (1.0 + math.exp(-s0))
    assert abs(out[0, 0, 0] - w0) < 1e-15
    assert abs(out[0, 0, 1] - (1.0 - w0)) < 1e-15
    assert np.all(out[0, 0, 2:] == 0.0)


def test_explicit_scale_equals_scaled_query(rng):
    B, hkv, T, d = 1, 1, 20, 16
    k, v = _contig(rng, B, hkv, T, d)
    q = rng.standard_normal((B, 1, d)).astype(np.float32)
    default = decode_attention(q * 2, k, v, [T])
    explicit = decode_attention(q, k, v, [T], scale=2.0 / math.sqrt(d))
    assert np.array_equal(default, explicit)


def test_dominant_key_returns_its_value(rng):
    """One key with a score gap >= 40 over the rest: the output is that row up to T·e^-40."""
    B, hkv, T, d = 1, 1, 300, 8
    k, v = _contig(rng, B, hkv, T, d)
    k[:] *= 0.01
    q = np.zeros((B, 1, d), dtype=np.float32)
    q[0, 0, 3] = 1.0
    k[0, 123, 0, 3] = 40.0 * math.sqrt(d) + 1.0
    out = decode_attention(q, k, v, [T])
    np.testing.assert_allclose(out[0, 0], v[0, 123, 0], rtol=0, atol=T * math.exp(-40) * 10)


def test_position_permutation_invariance(rng):
    B, hkv, T, d = 1, 2, 64, 16
    k, v = _contig(rng, B, hkv, T, d)
    q = (rng.standard_normal((B, 4, d)) * 3).astype(np.float32)
    perm = rng.permutation(T)
    a = decode_attention(q, k, v, [T])
    b = decode_attention(q, k[:, perm], v[:, perm], [T])
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    # permuting K alone must change the answer (K and V stay paired per position)
    c = decode_attention(q, k[:, perm], v, [T])
    assert np.max(np.abs(a - c)) > 1e-3


def test_gqa_equals_mha_on_repeated_kv_heads(rng):
    """Query head h reads KV head h // g: GQA equals MHA with each KV head repeated g times."""
    B, hkv, g, T, d = 2, 3, 4, 29, 16
    k, v = _contig(rng, B, hkv, T, d)
    q = rng.standard_normal((B, hkv * g, d)).astype(np.float32)
    gqa = decode_attention(q, k, v, [T, T - 5])
    mha = decode_attention(q, np.repeat(k, g, axis=2), np.repeat(v, g, axis=2), [T, T - 5])
    assert np.array_equal(gqa, mha)


def test_head_grouping_is_contiguous(rng):
    """With KV head j holding identical value rows c_j, query head h must return c_{h // g}."""
    B, hkv, g, T, d = 1, 4, 2, 10, 8
    k, _ = _contig(rng, B, hkv, T, d)
    const = np.arange(hkv, dtype=np.float32)[None, None, :, None] + 1
    v = np.broadcast_to(const, (B, T, hkv, d)).astype(np.float32)
    q = rng.standard_normal((B, hkv * g, d)).astype(np.float32)
    out = decode_attention(q, k, v, [T])
    for h in range(hkv * g):
        np.testing.assert_allclose(out[0, h], h // g + 1, rtol=1e-13)


def test_paged_gather_equals_contiguous(rng):
    """Scatter contiguous sequences into randomly permuted 16-token blocks (Ch. 19 §19.7.3)."""
    B, hkv, d, bs = 3, 2, 16, 16
    lens = [40, 16, 7]
    T = max(lens)
    k, v = _contig(rng, B, hkv, T, d)
    q = rng.standard_normal((B, 4, d)).astype(np.float32)
    nblk = [(t + bs - 1) // bs for t in lens]
    perm = rng.permutation(sum(nblk) + 2)
    kp = np.full((len(perm), bs, hkv, d), np.nan, dtype=np.float32)
    vp = np.full_like(kp, np.nan)
    table = np.full((B, max(nblk)), perm[-1])
    off = 0
    for b in range(B):
        for j in range(nblk[b]):
            p = perm[off + j]
            table[b, j] = p
            n = min(bs, lens[b] - j * bs)
            kp[p, :n] = k[b, j * bs:j * bs + n]
            vp[p, :n] = v[b, j * bs:j * bs + n]
        off += nblk[b]
    contiguous = decode_attention(q, k, v, lens)
    paged = decode_attention(q, kp, vp, lens, table, block_size=bs)
    assert np.array_equal(contiguous, paged)
    assert np.all(np.isfinite(paged))


def test_empty_context_gives_zero_row(rng):
    k, v = _contig(rng, 2, 1, 5, 8)
    q = rng.standard_normal((2, 1, 8)).astype(np.float32)
    out = decode_attention(q, k, v, [0, 5])
    assert np.all(out[0] == 0.0)
    assert np.any(out[1] != 0.0)


def test_final_rounding_is_round_to_nearest_even():
    x = np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, -(1.0 + 2.0 ** -24)])
    r = round_to_f32(x)
    assert r.dtype == np.float32
    assert r[0] == np.float32(1.0)                     # tie -> even
    assert r[1] == np.float32(1.0 + 2.0 ** -22)        # tie -> even (up)
    assert r[2] == np.float32(-1.0)


# ---------------------------------------------------------------------------------------------
# independent pure-Python implementation


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("paged", [False, True])
def test_numpy_oracle_matches_pure_python_fsum(rng, bf16, paged):
    B, hkv, g, d, bs = 2, 2, 2, 8, 16
    lens = [23, 9]
    T = max(lens)
    k, v = _contig(rng, B, hkv, T, d)
    q = (rng.standard_normal((B, hkv * g, d)) * 2).astype(np.float32)
    if bf16:
        k, v, q = _to_bf16_bits(k), _to_bf16_bits(v), _to_bf16_bits(q)
    table = None
    if paged:
        nblk = [(t + bs - 1) // bs for t in lens]
        perm = rng.permutation(sum(nblk))
        kp = np.zeros((len(perm), bs, hkv, d), dtype=k.dtype)
        vp = np.zeros_like(kp)
        table = np.zeros((B, max(nblk)), dtype=np.int64)
        off = 0
        for b in range(B):
            for j in range(nblk[b]):
                p = perm[off + j]
                table[b, j] = p
                n = min(bs, lens[b] - j * bs)
                kp[p, :n] = k[b, j * bs:j * bs + n]
                vp[p, :n] = v[b, j * bs:j * bs + n]
            off += nblk[b]
        k, v = kp, vp
    ref = decode_attention(q, k, v, lens, table, block_size=bs if paged else None)
    alt = np.array(decode_attention_fsum(q.tolist(), k.tolist(), v.tolist(), lens,
                                         None if table is None else table.tolist(),
                                         block_size=bs if paged else None, bf16=bf16))
    np.testing.assert_allclose(ref, alt, rtol=1e-13, atol=1e-15)


def test_numpy_oracle_matches_fsum_at_moderate_length(rng):
    """A longer row (T = 1500) keeps the oracle's summation error negligible."""
    B, hkv, T, d = 1, 1, 1500, 32
    k, v = _contig(rng, B, hkv, T, d)
    q = (rng.standard_normal((B, 1, d)) * 3).astype(np.float32)
    ref = decode_attention(q, k, v, [T])
    alt = np.array(decode_attention_fsum(q.tolist(), k.tolist(), v.tolist(), [T]))
    np.testing.assert_allclose(ref, alt, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------------------------
# appending the new token's K/V (the step before attention)


def test_append_places_rows_exactly_and_nowhere_else(rng):
    from oracle import append_kv, logical_rows
    B, hkv, d, bs = 3, 2, 8, 16
    nblk = 7
    cache = rng.standard_normal((nblk, bs, hkv, d)).astype(np.float32)
    table = np.array([[4, 1, 6], [0, 2, 6], [3, 5, 6]])
    new = rng.standard_normal((B, hkv, d)).astype(np.float32)
    pos = [17, 0, -1]  # sequence 2 appends nothing
    out = append_kv(cache, new, pos, table, block_size=bs)
    changed = np.argwhere(np.any(out != cache, axis=(2, 3)))
    assert sorted(map(tuple, changed)) == [(0, 0), (1, 1)]  # (block 1, slot 1) and (block 0, slot 0)
    for b in (0, 1):
        rows = logical_rows(out, table, b, 0, pos[b] + 1, bs)
        np.testing.assert_array_equal(rows[pos[b]], new[b, 0].astype(np.float64))
    assert np.array_equal(cache[3:], out[3:])


def test_append_contiguous_and_capacity(rng):
    from oracle import append_kv
    cache = np.zeros((2, 10, 1, 4), dtype=np.uint16)
    new = np.arange(8, dtype=np.uint16).reshape(2, 1, 4) + 1
    out = append_kv(cache, new, [9, 10], capacity=10)  # position 10 is past the capacity
    assert np.array_equal(out[0, 9, 0], [1, 2, 3, 4]) and not out[1].any()
    assert out[0, :9].sum() == 0


def test_append_then_attend_equals_attention_over_concatenated_rows(rng):
    """Appending then attending over T+1 positions is attention over the old rows plus the new
    one, assembled by hand (independent of the block translation)."""
    from oracle import append_kv
    B, hkv, d, bs, T = 1, 1, 16, 16, 20
    k_old = rng.standard_normal((T, d)).astype(np.float32)
    v_old = rng.standard_normal((T, d)).astype(np.float32)
    k_new = rng.standard_normal((B, hkv, d)).astype(np.float32)
    v_new = rng.standard_normal((B, hkv, d)).astype(np.float32)
    table = np.array([[2, 0]])
    kc = np.full((3, bs, hkv, d), np.nan, dtype=np.float32)
    vc = np.full_like(kc, np.nan)
    for t in range(T):
        kc[table[0, t // bs], t % bs, 0] = k_old[t]
        vc[table[0, t // bs], t % bs, 0] = v_old[t]
    kc = append_kv(kc, k_new, [T], table, block_size=bs)
    vc = append_kv(vc, v_new, [T], table, block_size=bs)
    q = rng.standard_normal((B, 1, d)).astype(np.float32)
    got = decode_attention(q, kc, vc, [T + 1], table, block_size=bs)
    keys = np.concatenate([k_old, k_new[0]], axis=0).astype(np.float64)
    vals = np.concatenate([v_old, v_new[0]], axis=0).astype(np.float64)
    s = (keys @ q[0, 0].astype(np.float64)) / math.sqrt(d)
    w = np.exp(s - s.max())
    np.testing.assert_allclose(got[0, 0], (w @ vals) / w.sum(), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------------------------
# sliding window and attention sinks (Ch. 19 §19.4.3)


def test_attended_positions_sets():
    from oracle import attended_positions
    assert attended_positions(10).tolist() == list(range(10))
    assert attended_positions(10, 3).tolist() == [7, 8, 9]
    assert attended_positions(10, 3, 2).tolist() == [0, 1, 7, 8, 9]
    assert attended_positions(10, 8, 4).tolist() == list(range(10))      # overlap: each once
    assert attended_positions(3, 5, 4).tolist() == [0, 1, 2]
    assert attended_positions(10, 0, 2).tolist() == [0, 1]
    assert attended_positions(0, 4, 4).tolist() == []


def test_window_of_one_returns_the_last_value_row(rng):
    k, v = _contig(rng, 2, 2, 30, 8)
    q = rng.standard_normal((2, 4, 8)).astype(np.float32)
    out = decode_attention(q, k, v, [30, 12], window=1)
    for b, t in ((0, 29), (1, 11)):
        for h in range(4):
            assert np.array_equal(out[b, h], v[b, t, h // 2].astype(np.float64))


def test_window_covering_everything_equals_full_attention(rng):
    k, v = _contig(rng, 2, 1, 40, 16)
    q = (rng.standard_normal((2, 2, 16)) * 2).astype(np.float32)
    full = decode_attention(q, k, v, [40, 25])
    assert np.array_equal(decode_attention(q, k, v, [40, 25], window=40, num_sinks=3), full)
    assert np.array_equal(decode_attention(q, k, v, [40, 25], window=1000), full)


def test_sinks_plus_window_equal_attention_over_the_kept_rows(rng):
    """Attention restricted to sinks + window equals full attention over a cache that holds only
    those rows, assembled by hand."""
    B, hkv, T, d = 1, 2, 50, 16
    k, v = _contig(rng, B, hkv, T, d)
    q = (rng.standard_normal((B, 4, d)) * 2).astype(np.float32)
    kept = list(range(4)) + list(range(T - 9, T))
    got = decode_attention(q, k, v, [T], window=9, num_sinks=4)
    want = decode_attention(q, k[:, kept], v[:, kept], [len(kept)])
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-15)


def test_windowed_numpy_oracle_matches_fsum(rng):
    B, hkv, T, d = 2, 2, 45, 8
    k, v = _contig(rng, B, hkv, T, d)
    q = (rng.standard_normal((B, 4, d)) * 2).astype(np.float32)
    for window, sinks in ((7, 0), (7, 3), (20, 30)):
        ref = decode_attention(q, k, v, [45, 33], window=window, num_sinks=sinks)
        alt = np.array(decode_attention_fsum(q.tolist(), k.tolist(), v.tolist(), [45, 33],
                                             window=window, num_sinks=sinks))
        np.testing.assert_allclose(ref, alt, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------------------------
# γ-query verification attention (Ch. 19 §19.8)


def _masked_matrix_attention(q, keys, values, scale, gamma, window=None, sinks=0):
    """Causal attention written as one masked score matrix (the prefill-style form): S = scale ·
    Q Kᵀ over all T positions, entries a query may not see set to -inf, row-wise softmax, times
    V. q: [γ, d]; keys/values: [T, d] fp64."""
    T = keys.shape[0]
    s = scale * (q @ keys.T)
    t = np.arange(T)[None, :]
    last = (T - gamma + np.arange(gamma))[:, None]       # position of query j
    visible = t <= last
    if window is not None:
        visible &= (t < sinks) | (t > last - window)
    s = np.where(visible, s, -np.inf)
    out = np.zeros((gamma, values.shape[1]))
    for j in range(gamma):
        if not visible[j].any():
            continue
        w = np.exp(s[j] - s[j].max())
        out[j] = (w @ values) / w.sum()
    return out


def test_one_query_is_plain_decode(rng):
    from oracle import verify_attention
    k, v = _contig(rng, 2, 2, 33, 16)
    q = rng.standard_normal((2, 1, 4, 16)).astype(np.float32)
    got = verify_attention(q, k, v, [33, 9])
    assert np.array_equal(got[:, 0], decode_attention(q[:, 0], k, v, [33, 9]))


@pytest.mark.parametrize("window,sinks", [(None, 0), (5, 0), (6, 2), (40, 3)])
def test_verification_equals_the_masked_matrix_form(rng, window, sinks):
    """Per-query truncated decode (the oracle) against the single masked score matrix, on a
    paged GQA cache; keys/values for the matrix form are gathered by hand."""
    from oracle import verify_attention
    B, gamma, hkv, g, d, bs = 2, 5, 2, 3, 16, 16
    lens = [37, 6]
    nblk = 6
    kc = rng.standard_normal((nblk, bs, hkv, d)).astype(np.float32)
    vc = rng.standard_normal((nblk, bs, hkv, d)).astype(np.float32)
    table = np.array([[5, 0, 3], [2, 4, 1]])
    q = (rng.standard_normal((B, gamma, hkv * g, d)) * 2).astype(np.float32)
    got = verify_attention(q, kc, vc, lens, table, block_size=bs, window=window, num_sinks=sinks)
    for b, T in enumerate(lens):
        for kvh in range(hkv):
            keys = np.stack([kc[table[b, t // bs], t % bs, kvh] for t in range(T)]).astype(np.float64)
            vals = np.stack([vc[table[b, t // bs], t % bs, kvh] for t in range(T)]).astype(np.float64)
            for i in range(g):
                h = kvh * g + i
                want = _masked_matrix_attention(q[b, :, h].astype(np.float64), keys, vals,
                                                1 / math.sqrt(d), gamma, window, sinks)
                np.testing.assert_allclose(got[b, :, h], want, rtol=1e-13, atol=1e-15)


def test_later_positions_do_not_reach_earlier_queries(rng):
    """Changing the K/V of the last position changes only the last query's output."""
    from oracle import verify_attention
    k, v = _contig(rng, 1, 1, 20, 8)
    q = rng.standard_normal((1, 4, 2, 8)).astype(np.float32)
    a = verify_attention(q, k, v, [20])
    k2, v2 = k.copy(), v.copy()
    k2[0, 19] += 3.0
    v2[0, 19] -= 2.0
    b = verify_attention(q, k2, v2, [20])
    assert np.array_equal(a[0, :3], b[0, :3])
    assert not np.allclose(a[0, 3], b[0, 3])


def test_queries_shorter_than_the_draft_give_zero_rows(rng):
    from oracle import verify_attention
    k, v = _contig(rng, 1, 1, 8, 8)
    q = rng.standard_normal((1, 5, 1, 8)).astype(np.float32)
    out = verify_attention(q, k, v, [3])                 # T = 3 < γ = 5
    assert not out[0, :2].any()                          # T_j = -1, 0
    np.testing.assert_array_equal(out[0, 2, 0], v[0, 0, 0].astype(np.float64))  # T_j = 1


def test_append_many_rows_equals_appending_them_one_by_one(rng):
    from oracle import append_kv
    B, n, hkv, d, bs = 2, 3, 2, 4, 16
    cache = rng.standard_normal((5, bs, hkv, d)).astype(np.float32)
    table = np.array([[3, 1], [0, 4]])
    new = rng.standard_normal((B, n, hkv, d)).astype(np.float32)
    pos = [14, 30]                                     # sequence 0 crosses a block edge
    got = append_kv(cache, new, pos, table, block_size=bs)
    want = cache
    for i in range(n):
        want = append_kv(want, new[:, i], [p + i for p in pos], table, block_size=bs)
    assert np.array_equal(got, want)
    assert np.array_equal(got[1, 0], new[0, 2]) and np.array_equal(got[4, 15], new[1, 1])
