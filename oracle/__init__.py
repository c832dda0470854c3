"""CPU fp64 oracle for single-token decode attention (test infrastructure).

This package is test infrastructure. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product package
``kv_cache_decode_split_amd`` never imports it, and the two share no code: no kernels, headers,
helpers, tables, constants or pre/post-processing. Only the seeded input generators
(``kv_cache_decode_split_amd.workloads``, which hold none of the method's arithmetic) feed both.

Modules
-------
decode_attention
    The plain definition: materialised scores, max-subtracted softmax, weighted sum of V.
online_softmax
    The blockwise running-(m, l, O) recurrence and the merge of two running states, written in
    the order the pages give them. Used to pin the exactness claim by brute force and as the
    reference for the GPU merge step.
fsum_reference
    A second, pure-Python (math.fsum) implementation of the plain definition for tiny shapes.
kv_append
    Writing new tokens' K/V rows into a contiguous or block-table cache (the step before
    attention).
verify_attention
    γ new query tokens per sequence attending causally among themselves (the target model's
    check of a speculative-decoding draft).
position_scores
    The attention weight each cached position receives in a decode step, summed over the query
    heads of its KV head (the per-entry score eviction ranks by).
evict_select
    Budgeted KV eviction selection: the current position of every (layer, head) kept, the rest
    ranked in one global pool by (−score, layer, head, token) and the first M − L·H kept.

Every function here is pinned by ``tests/test_oracle_*.py`` against closed forms, invariants,
brute force and the independent pure-Python implementation (no function is "parity unpinned").
"""

from .decode_attention import (  # noqa: F401
    widen,
    logical_rows,
    attended_positions,
    stable_softmax,
    attend_one,
    decode_attention,
    round_to_f32,
)
from .online_softmax import (  # noqa: F401
    EMPTY_STATE,
    block_state,
    online_softmax,
    merge_states,
    merge_many,
    finalize_state,
)
from .fsum_reference import decode_attention_fsum  # noqa: F401
from .kv_append import append_kv  # noqa: F401
from .verify_attention import verify_attention  # noqa: F401
from .evict_select import evict_select  # noqa: F401
from .position_scores import position_scores  # noqa: F401
