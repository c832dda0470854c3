"""Byte, FLOP, intensity and roofline accounting for decode attention.

Host-side bookkeeping used by the bench and its tests; it never touches the data path.

Sources, by page title and section:

* Appendix "Inference Fundamentals" (推理基础), Eq. 3: KV-cache size
  M_KV = 2 · N_L · d · S · B · s_elem (keys and values, hidden size d).
* Ch. 10 "System Model of Throughput and Latency" (第十章 吞吐与延迟的系统模型):
  §1 metric table (decode aggregate throughput = tokens of the step / step time; per-sequence
  rate = 1 / step time); §2 roofline time bound t >= max(F / C_peak, D / beta_peak) and the
  per-kernel sum; §4 dense-decode KV read traffic 2·L·B·T·d_kv·b_kv counted over unique KV
  elements under GQA; §5 decode-attention intensity 4·L·B·d_q·T / (2·L·B·T·d_kv·b_kv)
  = 2·h_q / (h_kv·b_kv).
* Ch. 19 "Inference Systems and Performance Engineering" (第19章 推理系统与性能工程):
  §19.2.1 ridge point I* = P_peak / BW; §19.2.2 two FLOPs per multiply-add; §19.3.2 decode
  step bound for a 7B-class model (weights plus KV read once per step); §19.4.2 KV bytes per
  token 2 · L · h · 2 (fp16); self-test Q1 (compare the memory and compute time bounds).

Conventions (readings): FLOPs count 2 per multiply-add, so decode attention costs
4 · h_q · d per attended (sequence, position) pair (QKᵀ and PV); the KV metric counts reads of
the positions attended (the new token's write belongs to the append step that precedes the
kernel); "unique" means each K/V element once, however many query heads share it.
"""

from __future__ import annotations

from typing import Iterable, Union

__all__ = [
    "attended_length",
    "verify_attention_flops",
    "MI355X_HBM_PEAK_GBPS",
    "kv_cache_bytes_eq3",
    "kv_bytes_per_token",
    "unique_kv_read_bytes",
    "unique_kv_bytes_per_position",
    "decode_attention_flops",
    "decode_attention_intensity",
    "ridge_point",
    "roofline_time",
    "roofline_time_sum",
    "aggregate_tokens_per_s",
    "per_sequence_tokens_per_s",
    "decode_step_bandwidth_bound",
]

# MI355X HBM3E peak (published figure), in GB/s (1 GB = 1e9 bytes).
MI355X_HBM_PEAK_GBPS = 8000.0

Lengths = Union[int, Iterable[int]]


def _total(lengths: Lengths, batch: int | None) -> int:
    if isinstance(lengths, int):
        if batch is None:
            raise ValueError("a single context length needs the batch size")
        return lengths * batch
    return int(sum(int(t) for t in lengths))


def kv_cache_bytes_eq3(num_layers: int, hidden: int, seq_len: int, batch: int, elem_bytes: int) -> int:
    """Appendix "Inference Fundamentals", Eq. 3: 2 · N_L · d · S · B · s_elem bytes."""
    return 2 * num_layers * hidden * seq_len * batch * elem_bytes


def kv_bytes_per_token(num_layers: int, hidden: int, elem_bytes: int = 2) -> int:
    """Ch. 19 §19.4.2: every layer keeps one K and one V vector of the hidden size per token."""
    return 2 * num_layers * hidden * elem_bytes


def unique_kv_bytes_per_position(num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes of K and V for one (sequence, position) over all KV heads: 2 · d_kv · b_kv."""
    return 2 * num_kv_heads * head_dim * elem_bytes


def attended_length(length: int, window: int | None = None, num_sinks: int = 0,
                    num_queries: int = 1) -> int:
    """Positions a decode step attends to in a sequence of ``length`` positions: all of them, or
    with a window W the union of the first ``num_sinks`` and the last W positions (Ch. 19 §19.4.3
    sliding window with attention sinks). These are the positions whose KV the step reads.

    With ``num_queries`` = γ query tokens (the last γ positions, each attending to its own
    prefix, Ch. 19 §19.8) the count is that of the union of the γ tokens' positions: with a
    window, the first ``num_sinks`` and the last W + γ - 1 positions."""
    length = max(int(length), 0)
    if window is None:
        return length
    span = int(window) + max(int(num_queries), 1) - 1
    return min(length, min(int(num_sinks), length) + min(span, length))


def verify_attention_flops(length: int, num_q_heads: int, head_dim: int, num_queries: int,
                           window: int | None = None, num_sinks: int = 0) -> int:
    """FLOPs of the γ query tokens of one sequence of ``length`` cached positions: token j
    attends to the first length - γ + 1 + j positions (windowed as for one token), at
    4 · h_q · d FLOPs per attended position (QKᵀ and PV, 2 FLOPs per multiply-add)."""
    total = 0
    for j in range(num_queries):
        visible = int(length) - num_queries + 1 + j
        if visible > 0:
            total += attended_length(visible, window, num_sinks)
    return 4 * num_q_heads * head_dim * total


def unique_kv_read_bytes(lengths: Lengths, num_kv_heads: int, head_dim: int, elem_bytes: int,
                         batch: int | None = None, num_layers: int = 1) -> int:
    """Ch. 10 §4 old-KV read term 2 · L · Σ_b T_b · d_kv · b_kv (each element counted once)."""
    return num_layers * _total(lengths, batch) * unique_kv_bytes_per_position(
        num_kv_heads, head_dim, elem_bytes)


def decode_attention_flops(lengths: Lengths, num_q_heads: int, head_dim: int,
                           batch: int | None = None, num_layers: int = 1) -> int:
    """Ch. 10 §5 numerator 4 · L · d_q · Σ_b T_b (QKᵀ and PV, 2 FLOPs per multiply-add)."""
    return 4 * num_layers * num_q_heads * head_dim * _total(lengths, batch)


def decode_attention_intensity(num_q_heads: int, num_kv_heads: int, elem_bytes: float) -> float:
    """Ch. 10 §5: I_attn = 2 · h_q / (h_kv · b_kv) FLOP per byte of unique KV."""
    return 2.0 * num_q_heads / (num_kv_heads * elem_bytes)


def ridge_point(peak_flops: float, bandwidth: float) -> float:
    """Ch. 19 §19.2.1: I* = P_peak / BW."""
    return peak_flops / bandwidth


def roofline_time(flops: float, nbytes: float, peak_flops: float, bandwidth: float) -> float:
    """Ch. 10 §2: t >= max(F / C_peak, D / beta_peak), in seconds."""
    return max(flops / peak_flops, nbytes / bandwidth)


def roofline_time_sum(kernels, exposed_other: float = 0.0) -> float:
    """Ch. 10 §2 per-kernel sum: Σ_j max(F_j / C_j, D_j / beta_j) + exposed other time.

    ``kernels`` is an iterable of (flops, bytes, peak_flops, bandwidth).
    """
    return sum(max(f / c, d / b) for f, d, c, b in kernels) + exposed_other


def aggregate_tokens_per_s(batch: int, step_seconds: float) -> float:
    """Ch. 10 §1: decode aggregate throughput = B / t for one token per sequence per step."""
    return batch / step_seconds


def per_sequence_tokens_per_s(step_seconds: float) -> float:
    """Ch. 10 §1: per-sequence rate = 1 / t."""
    return 1.0 / step_seconds


def decode_step_bandwidth_bound(num_params: float, num_layers: int, hidden: int, seq_len: int,
                                bandwidth: float, elem_bytes: int = 2) -> float:
    """Ch. 19 §19.3.2: one decode step reads all weights and the K/V of every cached token.

    bytes = b · P + 2 · b · L · h · s; the bound is bytes / bandwidth (seconds).
    """
    nbytes = elem_bytes * num_params + 2 * elem_bytes * num_layers * hidden * seq_len
    return nbytes / bandwidth
