"""GPU parity at the size limits of the planner.

* The longest sequence the oracle still checks in seconds: one sequence of 4,194,304 positions
  (1 GiB each of K and V, paged in 16-token blocks, 4 sink keys), planned as 512 splits of 8192
  positions; every head is compared with the fp64 oracle.
* The split cap: one sequence of 33,554,432 positions (8 GiB each of K and V) plans exactly the
  maximum of 4096 splits, and the merge combines all of them. Checked by a property that holds
  at any size (the pages fix it: when every value row is the same, the output is that row,
  whatever the weights), on the rows-mode kernel (group 16) and the one-token kernel (group 1).
"""

import pytest
import torch

from kv_cache_decode_split_amd import workloads as W
from tests.gpu_helpers import announce, check_close, oracle_full, require_gpu, run

pytestmark = pytest.mark.gpu


def _free(w):
    del w
    torch.cuda.empty_cache()


def test_longest_sequence_matches_oracle():
    K = require_gpu()
    T = 1 << 22
    spec = W.WorkloadSpec(name="long", batch=1, num_q_heads=8, num_kv_heads=1, head_dim=128,
                          ctx=(T,), paged=True, block_size=16, num_sinks=4, seed=9101)
    announce(f"limits: one sequence of {T} positions")
    w = W.make_workload(spec, device="cuda")
    try:
        out = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")
        assert K.decode_call_for(w, out).plan()["num_splits"] == 512
        check_close(run(w).cpu().numpy(), oracle_full(w), f"T={T}")
    finally:
        _free(w)


@pytest.mark.parametrize("num_q_heads", [16, 1])
def test_split_cap_with_equal_value_rows(num_q_heads):
    K = require_gpu()
    T = 1 << 25
    spec = W.WorkloadSpec(name="cap", batch=1, num_q_heads=num_q_heads, num_kv_heads=1,
                          head_dim=128, ctx=(T,), paged=True, block_size=16, seed=9102)
    announce(f"limits: {T} positions, 4096 splits, group {num_q_heads}")
    w = W.make_workload(spec, device="cuda")
    try:
        live = w.block_table[0].long()
        row = w.v_cache[live[0], 0, 0].clone()          # head-major blocks [N, h_kv, 16, d]
        w.v_cache[live] = row                            # every attended value row equal
        out = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")
        plan = K.decode_call_for(w, out).plan()
        assert plan["num_splits"] == 4096 and plan["split_len"] == 8192
        got = run(w)[0].double().cpu().numpy()           # [h_q, d]
        want = row.float().double().cpu().numpy()[None].repeat(num_q_heads, 0)
        check_close(got, want, f"T={T} S=4096 g={num_q_heads}")
        assert abs(got - want).max() <= 1e-4 * abs(want).max()
    finally:
        _free(w)
