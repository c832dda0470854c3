"""GPU parity of the budgeted eviction selection against the oracle ``oracle.evict_select``.

The result is a set (unique, rule 4 of the page), so the GPU mask must equal the oracle's bit
for bit. Full-size workloads are checked against the oracle as well and, independently of it,
by the properties the ranking fixes at any size: the kept count, every kept pool score at least
every dropped one, and among entries equal to the boundary score the kept ones before the
dropped ones in (layer, head, position) order.
"""

import random

import numpy as np
import pytest
import torch

from kv_cache_decode_split_amd import workloads as W
from tests.gpu_helpers import announce, require_gpu

pytestmark = pytest.mark.gpu


def _evict():
    require_gpu()
    from kv_cache_decode_split_amd import kv_evict
    return kv_evict


def _oracle(scores, budget, current):
    from oracle import evict_select
    return evict_select(scores.cpu().numpy(), budget, current)


def _check_properties(scores_np, keep_np, budget, current):
    L, H, N = scores_np.shape
    pool = np.ones((L, H, N), dtype=bool)
    pool[:, :, current] = False
    assert keep_np[:, :, current].all()
    free = min(max(budget - L * H, 0), L * H * (N - 1))
    kept = keep_np & pool
    dropped = ~keep_np & pool
    assert int(kept.sum()) == free
    if free == 0 or not dropped.any():
        return
    s = scores_np.astype(np.float64)
    lo = s[kept].min()
    assert lo >= s[dropped].max()
    flat = np.arange(L * H * N).reshape(L, H, N)
    tie_kept = flat[kept & (s == lo)]
    tie_dropped = flat[dropped & (s == lo)]
    if tie_kept.size and tie_dropped.size:
        assert tie_kept.max() < tie_dropped.min()


def _run_case(E, scores, budget, current, label):
    announce(f"evict {label} shape={tuple(scores.shape)} stride={scores.stride()} M={budget} C={current}")
    counts = torch.full(scores.shape[:2], -1, dtype=torch.int32, device=scores.device)
    keep = E.kv_evict_select(scores, budget, current, kept_per_row=counts)
    torch.cuda.synchronize()
    got = keep.cpu().numpy().astype(bool)
    want = _oracle(scores, budget, current if current is not None else scores.shape[2] - 1)
    assert np.array_equal(got, want), f"{label}: {int((got != want).sum())} entries differ"
    assert np.array_equal(counts.cpu().numpy(), want.sum(axis=2)), f"{label}: per-row counts"
    return keep


SMALL = [
    # (L, H, N, kind, budget as a function of (L, H, N), current, row_stride)
    (2, 2, 4, "levels", lambda L, H, N: 10, 3, None),
    (1, 1, 1, "normal", lambda L, H, N: 3, 0, None),            # N = 1: only the current position
    (3, 2, 7, "normal", lambda L, H, N: L * H + 5, 2, None),    # N not a multiple of 4
    (2, 3, 16, "levels", lambda L, H, N: L * H + 1, 0, 21),     # one free slot, strided rows
    (2, 3, 16, "levels", lambda L, H, N: L * H * N - 1, 15, None),   # all but one
    (4, 8, 300, "lognormal", lambda L, H, N: L * H * N // 3, 299, None),
    (4, 8, 300, "equal", lambda L, H, N: L * H * N // 3, 5, None),   # every score ties
    (4, 8, 301, "levels", lambda L, H, N: L * H * N // 2, 100, 304),
    (1, 4, 5000, "normal", lambda L, H, N: 7000, 4999, None),
    (4, 8, 5000, "lognormal", lambda L, H, N: L * H * N // 10, 4999, None),   # many workgroups
    (4, 8, 5000, "levels", lambda L, H, N: L * H * N // 10, 17, None),
    (4, 8, 5000, "equal", lambda L, H, N: L * H * N // 2, 2500, 5004),
    (2, 2, 8, "normal", lambda L, H, N: 0, 7, None),            # budget 0
    (2, 2, 8, "normal", lambda L, H, N: L * H, 7, None),        # exactly the current positions
    (2, 2, 8, "normal", lambda L, H, N: L * H * N, 7, None),    # everything
    (2, 2, 8, "normal", lambda L, H, N: 10**12, 0, None),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}x{c[1]}x{c[2]}-{c[3]}-{i}" for i, c in enumerate(SMALL)])
def test_small_selections_match_oracle(case):
    E = _evict()
    L, H, N, kind, budget_of, current, stride = case
    scores = W.make_scores(L, H, N, kind, seed=L * 100 + N, device="cuda", row_stride=stride)
    _run_case(E, scores, budget_of(L, H, N), current, f"{kind}")


def test_signed_zeros_and_infinities():
    E = _evict()
    vals = torch.tensor([0.0, -0.0, float("inf"), float("-inf"), 1.0, -1.0, 0.0, -0.0],
                        dtype=torch.float32)
    g = torch.Generator().manual_seed(3)
    idx = torch.randint(0, len(vals), (3, 5, 64), generator=g)
    scores = vals[idx].cuda()
    for M in (15, 16, 100, 500, 15 + 3 * 5 * 63 - 1):
        _run_case(E, scores, M, 10, "zeros-inf")


def _random_cases(n, seed=41):
    rnd = random.Random(seed)
    out = []
    for i in range(n):
        L, H = rnd.randint(1, 6), rnd.randint(1, 9)
        N = rnd.choice([1, 2, 3, 4, 5, 16, 63, 64, 100, 1023, 1024, 4097])
        stride = None if rnd.random() < 0.6 else N + rnd.choice([1, 3, 4, 8])
        kind = rnd.choice(["lognormal", "levels", "normal", "equal"])
        total = L * H * N
        budget = rnd.choice([0, L * H, L * H + 1, rnd.randint(0, total + 3), total - 1, total])
        out.append((L, H, N, stride, kind, max(budget, 0), rnd.randrange(N), 5000 + i))
    return out


RANDOM = _random_cases(40)


@pytest.mark.parametrize("case", RANDOM, ids=[f"r{i}" for i in range(len(RANDOM))])
def test_random_selections_match_oracle(case):
    E = _evict()
    L, H, N, stride, kind, budget, current, seed = case
    scores = W.make_scores(L, H, N, kind, seed=seed, device="cuda", row_stride=stride)
    _run_case(E, scores, budget, current, f"random {kind}")


def test_workspace_is_reused_across_calls_of_different_sizes():
    E = _evict()
    big = W.make_scores(8, 8, 2048, "lognormal", seed=7, device="cuda")
    small = W.make_scores(2, 4, 300, "levels", seed=8, device="cuda")
    from kv_cache_decode_split_amd.kv_evict import make_evict_params, kv_evict_workspace_size
    ws = torch.empty(kv_evict_workspace_size(make_evict_params(8, 8, 2048, 8 * 8 * 512)),
                     dtype=torch.uint8, device="cuda")
    ws.fill_(0xAB)  # contents need no initialisation
    for scores, M in ((big, 8 * 8 * 512), (small, 900), (big, 8 * 8 * 100), (small, 9)):
        keep = E.kv_evict_select(scores, M, workspace=ws)
        torch.cuda.synchronize()
        want = _oracle(scores, M, scores.shape[2] - 1)
        assert np.array_equal(keep.cpu().numpy().astype(bool), want)


def test_repeated_calls_are_identical():
    E = _evict()
    scores = W.make_scores(4, 8, 4096, "levels", seed=12, device="cuda")
    first = E.kv_evict_select(scores, 40000).clone()
    for _ in range(3):
        assert torch.equal(E.kv_evict_select(scores, 40000), first)


@pytest.mark.parametrize("name", ["E1", "E2"])
def test_full_size_selections(name):
    E = _evict()
    cfg = W.EVICT_PRESETS[name]
    L, H, N = cfg["num_layers"], cfg["num_heads"], cfg["num_tokens"]
    budget = int(cfg["budget_frac"] * L * H * N)
    announce(f"evict full {name} L={L} H={H} N={N} M={budget}")
    scores = W.make_scores(L, H, N, cfg["kind"], seed=cfg["seed"], device="cuda", sigma=cfg["sigma"])
    counts = torch.empty((L, H), dtype=torch.int32, device="cuda")
    keep = E.kv_evict_select(scores, budget, kept_per_row=counts)
    torch.cuda.synchronize()
    got = keep.cpu().numpy().astype(bool)
    s = scores.cpu().numpy()
    _check_properties(s, got, budget, N - 1)
    assert np.array_equal(counts.cpu().numpy(), got.sum(axis=2))
    if name == "E1":
        assert np.array_equal(got, _oracle(scores, budget, N - 1))
    del scores, keep
    torch.cuda.empty_cache()


def test_selection_over_a_billion_entries():
    """2^30 entries (16 layers x 16 heads x 4,194,304 positions; flat indices up to 2^30 in the
    keys, 16 GiB of candidate lists): checked on the GPU by the properties that fix the set
    (kept count, every kept pool score at least every dropped one, ties kept in index order)."""
    E = _evict()
    L, H, N = 16, 16, 1 << 22
    budget = L * H + (L * H * (N - 1)) // 7
    announce(f"evict 2^30 entries M={budget}")
    scores = W.make_scores(L, H, N, "lognormal", seed=2099, device="cuda")
    counts = torch.empty((L, H), dtype=torch.int32, device="cuda")
    keep = E.kv_evict_select(scores, budget, kept_per_row=counts).bool()
    try:
        assert keep[:, :, N - 1].all()
        assert torch.equal(counts, keep.sum(dim=2, dtype=torch.int32))
        pool_kept = keep.clone()
        pool_kept[:, :, N - 1] = False
        assert int(pool_kept.sum()) == budget - L * H
        inf = torch.tensor(float("inf"), device="cuda")
        lo = torch.where(pool_kept, scores, inf).min()
        hi = torch.where(keep, -inf, scores).max()
        assert float(lo) >= float(hi)
        if float(lo) == float(hi):
            flat = torch.arange(L * H * N, device="cuda").view(L, H, N)
            big = torch.tensor(L * H * N, device="cuda")
            last_kept = torch.where(pool_kept & (scores == lo), flat, -1).max()
            first_dropped = torch.where(~keep & (scores == lo), flat, big).min()
            assert int(last_kept) < int(first_dropped)
    finally:
        del scores, keep
        torch.cuda.empty_cache()


FALLBACK = [
    (4, 8, 300, "lognormal", 0.3, 299, None),
    (4, 8, 5000, "levels", 0.1, 17, None),
    (3, 5, 4097, "normal", 0.5, 100, 4100),     # strided rows
    (8, 8, 4096, "lognormal", 0.25, 4095, None),  # sampled in chunks (above 131072 entries)
]


@pytest.mark.parametrize("case", FALLBACK, ids=[f"fb{i}" for i in range(len(FALLBACK))])
def test_exact_fallback_matches_oracle(case, monkeypatch):
    """The exact path the final workgroup takes when k* lies outside the sampled band (forced
    here for every ranked call) gives the same mask."""
    E = _evict()
    L, H, N, kind, frac, current, stride = case
    monkeypatch.setenv("KV_EVICT_FORCE_FALLBACK", "1")
    scores = W.make_scores(L, H, N, kind, seed=N + L, device="cuda", row_stride=stride)
    _run_case(E, scores, int(frac * L * H * N), current, f"fallback {kind}")


def test_sample_unlike_the_rest_still_selects_exactly():
    """Scores whose sampled region differs from the rest (the first 1/64 of every row is large,
    the sampled chunks lie all over the array): the band may miss k*, and the result must still
    be the exact selection."""
    E = _evict()
    L, H, N = 8, 8, 8192
    scores = W.make_scores(L, H, N, "lognormal", seed=91, device="cuda")
    scores[:, :, : N // 64] += 1000.0
    for frac in (0.01, 0.1, 0.5):
        _run_case(E, scores, int(frac * L * H * N), N - 1, f"skewed {frac}")
