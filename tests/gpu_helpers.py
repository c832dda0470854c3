"""Shared helpers of the GPU tests: running the HIP path and the oracle on the same inputs.

The HIP path is always the C library through its ctypes binding; the expected values always
come from the fp64 oracle in ``oracle/`` on host copies of the same seeded inputs.
"""

from __future__ import annotations

import os
import sys

import numpy as np
import torch

from kv_cache_decode_split_amd import workloads as W

# Tolerance of the parity gate: max |gpu - ref| <= 5e-3 and max |gpu - ref| / max |ref| <= 1e-2,
# on the fp32 output (the stated target for bf16 or fp32 KV).
ATOL = 5e-3
RTOL_OF_MAX = 1e-2


def require_gpu():
    """Fail (never skip) when the device or the native library is missing."""
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    from kv_cache_decode_split_amd import kv_attn  # raises ImportError if the .so is missing
    return kv_attn


def loaded_native_libraries():
    """Paths of in-tree native libraries this process has mapped (evidence the HIP path ran)."""
    out = []
    with open(f"/proc/{os.getpid()}/maps") as f:
        for line in f:
            if "libkvattn.so" in line:
                out.append(line.split()[-1])
    return sorted(set(out))


def run(w: W.Workload, **kwargs) -> torch.Tensor:
    K = require_gpu()
    out = torch.full(w.q.shape, float("nan"), dtype=torch.float32, device=w.q.device)
    K.kv_attn_decode_workload(w, out, **kwargs)
    torch.cuda.synchronize()
    return out


def _window_kwargs(w: W.Workload) -> dict:
    """The workload's sliding window, in the oracle's terms (None = every position)."""
    if w.spec.window is None:
        return {}
    return dict(window=w.spec.window, num_sinks=w.spec.num_sinks)


def oracle_full(w: W.Workload, scale=None) -> np.ndarray:
    from oracle import decode_attention
    v = W.oracle_view(w)
    return decode_attention(v["q"], v["k_cache"], v["v_cache"], v["ctx_lens"], v["block_table"],
                            block_size=v["block_size"] if v["block_table"] is not None else None,
                            scale=scale, **_window_kwargs(w))


def oracle_rows(w: W.Workload, seqs, kv_heads=None, scale=None) -> np.ndarray:
    """Oracle output for the sequences ``seqs`` (and KV heads ``kv_heads``) only."""
    from oracle import decode_attention
    v = W.oracle_sample(w, seqs, kv_heads)
    return decode_attention(v["q"], v["k_cache"], v["v_cache"], v["ctx_lens"], v["block_table"],
                            block_size=v["block_size"] if v["block_table"] is not None else None,
                            scale=scale, **_window_kwargs(w))


def select_rows(out: torch.Tensor, w: W.Workload, seqs, kv_heads=None) -> np.ndarray:
    o = out[[int(s) for s in seqs]]
    if kv_heads is not None:
        g = w.spec.group
        heads = [kvh * g + j for kvh in kv_heads for j in range(g)]
        o = o[:, heads]
    return o.cpu().numpy().astype(np.float64)


def check_close(gpu: np.ndarray, ref: np.ndarray, label: str = ""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{label}: non-finite output"
    err = np.abs(gpu - ref)
    max_abs = float(err.max()) if err.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    rel = max_abs / scale if scale > 0 else max_abs
    print(f"[parity] {label} max_abs={max_abs:.3e} max_rel_of_max={rel:.3e}", file=sys.stderr)
    assert max_abs <= ATOL, f"{label}: max abs error {max_abs:.3e} > {ATOL}"
    assert rel <= RTOL_OF_MAX, f"{label}: max error / max |ref| = {rel:.3e} > {RTOL_OF_MAX}"
    return max_abs, rel


def announce(msg: str):
    """Name the case before a GPU step (flushed, so it survives an abrupt end)."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)
