"""Seeded planning cases shared by the ABI tests and the host sanitizer run.

Each case is a dict of ``make_params`` keyword arguments (the base problem of ``BASE`` with some
fields replaced) and, for the sweeps, the compute-unit count to plan for. Nothing here calls the
library.
"""

from __future__ import annotations

import numpy as np

# A paged head-major problem: 4 sequences, 32 query heads over 8 KV heads, d = 128.
BASE = dict(batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
            max_ctx_len=1000, num_blocks=300, k_strides=(8 * 16 * 128, 128, 16 * 128),
            v_strides=(8 * 16 * 128, 128, 16 * 128), max_blocks_per_seq=63)


def params_kwargs(**kw) -> dict:
    out = dict(BASE)
    out.update(kw)
    return out


def token_major(hkv, d=128, bs=16) -> dict:
    return dict(k_strides=(bs * hkv * d, hkv * d, d), v_strides=(bs * hkv * d, hkv * d, d))


def random_plan_cases(n=400, seed=17):
    """Shapes, windows, query tokens and CU counts: (kwargs, num_cus, label fields)."""
    rnd = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        B = int(rnd.integers(1, 200))
        hkv = int(rnd.choice([1, 2, 4, 8, 32]))
        g = int(rnd.choice([1, 2, 3, 4, 8, 16]))
        nq = int(rnd.choice([1, 1, 2, 4]))
        if nq * g > 32:
            nq = 1
        T = int(rnd.choice([1, 15, 16, 17, 300, 4096, 8191, 32768, 131072, 1 << 20]))
        W = int(rnd.choice([0, 0, 1, 64, 1000, 4096]))
        n_sinks = int(rnd.choice([0, 4, 100]))
        cus = int(rnd.choice([1, 64, 256, 304]))
        kw = params_kwargs(batch=B, num_q_heads=hkv * g, num_kv_heads=hkv, max_ctx_len=T,
                           max_blocks_per_seq=(T + 15) // 16, num_blocks=10**7, window=W or None,
                           num_sinks=n_sinks, num_queries=nq)
        cases.append((kw, cus, dict(B=B, hkv=hkv, g=g, nq=nq, T=T, W=W, n=n_sinks)))
    return cases


def random_token_major_cases(n=300, seed=23):
    """Token-major caches with h_kv a multiple of 4: (kwargs, num_cus, label fields)."""
    rnd = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        B = int(rnd.integers(1, 200))
        hkv = int(rnd.choice([4, 8, 12, 32]))
        g = int(rnd.choice([1, 2, 4, 8]))
        T = int(rnd.choice([1, 15, 17, 300, 4096, 32768, 131072, 1 << 20]))
        W = int(rnd.choice([0, 0, 64, 4096]))
        cus = int(rnd.choice([1, 64, 256, 304]))
        kw = params_kwargs(batch=B, num_q_heads=hkv * g, num_kv_heads=hkv, max_ctx_len=T,
                           max_blocks_per_seq=(T + 15) // 16, num_blocks=10**7, window=W or None,
                           num_sinks=4, **token_major(hkv))
        cases.append((kw, cus, dict(B=B, hkv=hkv, g=g, T=T, W=W)))
    return cases


# (replaced fields, expected status name) of problems the library must reject.
INVALID_PARAM_CASES = [
    (dict(batch=0), "KV_ATTN_ERR_SHAPE"),
    (dict(num_q_heads=30), "KV_ATTN_ERR_SHAPE"),              # not a multiple of h_kv
    (dict(num_q_heads=8 * 17), "KV_ATTN_ERR_UNSUPPORTED"),    # group 17 > 16
    (dict(batch=1 << 24, num_queries=2), "KV_ATTN_ERR_UNSUPPORTED"),  # 2^31 append pieces
    (dict(head_dim=96), "KV_ATTN_ERR_UNSUPPORTED"),
    (dict(q_dtype=5), "KV_ATTN_ERR_UNSUPPORTED"),
    (dict(k_strides=(8 * 16 * 128, 127, 16 * 128)), "KV_ATTN_ERR_UNSUPPORTED"),  # misaligned rows
    (dict(v_strides=(-1, 128, 16 * 128)), "KV_ATTN_ERR_SHAPE"),
    (dict(max_ctx_len=-1), "KV_ATTN_ERR_VALUE"),
    (dict(num_splits=-2), "KV_ATTN_ERR_VALUE"),
    (dict(scale=float("nan")), "KV_ATTN_ERR_VALUE"),
    (dict(num_blocks=0), "KV_ATTN_ERR_SHAPE"),
    (dict(window=64, num_sinks=-1), "KV_ATTN_ERR_VALUE"),
]

# Paged layout problems rejected before any device work (validate_layout).
INVALID_LAYOUT_CASES = [
    dict(block_size=24),                         # not a power of two
    dict(block_size=8, max_blocks_per_seq=200),  # below one 16-position tile
    dict(max_ctx_len=63 * 16 + 1),               # longer than the table
]
