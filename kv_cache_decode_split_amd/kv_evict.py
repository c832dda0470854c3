"""ctypes binding of the eviction-selection entry points declared in ``include/kv_evict.h``.

Argument marshalling only (tensor checks, raw pointers, torch's current stream); the selection
runs in the library's HIP kernels. Uses the library loaded by :mod:`kv_attn` (importing this
module raises ImportError when it has not been built).
"""

from __future__ import annotations

import ctypes
from typing import Optional

import torch

from .kv_attn import _check_device, _hold_for_stream, _lib, _stream_handle, KvAttnError, KV_ATTN_OK

__all__ = ["kv_evict_params", "make_evict_params", "kv_evict_workspace_size", "kv_evict_select",
           "EXPORTED_SYMBOLS"]

EXPORTED_SYMBOLS = ("kv_evict_workspace_size", "kv_evict_select")


class kv_evict_params(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("num_tokens", ctypes.c_int32),
        ("current", ctypes.c_int32),
        ("budget", ctypes.c_int64),
        ("row_stride", ctypes.c_int64),
    ]


_P = ctypes.POINTER(kv_evict_params)
_vp = ctypes.c_void_p
_lib.kv_evict_workspace_size.argtypes = [_P]
_lib.kv_evict_workspace_size.restype = ctypes.c_size_t
_lib.kv_evict_select.argtypes = [_vp, _vp, _vp, _P, _vp, ctypes.c_size_t, _vp]
_lib.kv_evict_select.restype = ctypes.c_int


def make_evict_params(num_layers: int, num_heads: int, num_tokens: int, budget: int,
                      current: Optional[int] = None, row_stride: Optional[int] = None) -> kv_evict_params:
    p = kv_evict_params()
    p.num_layers, p.num_heads, p.num_tokens = int(num_layers), int(num_heads), int(num_tokens)
    p.current = int(num_tokens) - 1 if current is None else int(current)
    p.budget = int(budget)
    p.row_stride = int(num_tokens) if row_stride is None else int(row_stride)
    return p


def kv_evict_workspace_size(p: kv_evict_params) -> int:
    return int(_lib.kv_evict_workspace_size(ctypes.byref(p)))


def kv_evict_select(scores: torch.Tensor, budget: int, current: Optional[int] = None, *,
                    keep: Optional[torch.Tensor] = None,
                    kept_per_row: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Mask of the entries that stay under a global budget (uint8 [L, H, N], 1 = stays).

    scores: fp32 device tensor [L, H, N] whose last axis is contiguous and whose (L, H) axes
    form equally spaced rows (e.g. a contiguous tensor, or a slice of a wider one along N).
    current: the current position (default N - 1). kept_per_row: optional int32 [L, H] output.
    """
    if scores.dim() != 3 or scores.dtype != torch.float32 or not scores.is_cuda:
        raise ValueError("scores must be an fp32 [L, H, N] tensor on a GPU")
    _check_device(scores, "scores")
    L, H, N = scores.shape
    if scores.stride(2) != 1 or (H > 1 and L > 1 and scores.stride(0) != H * scores.stride(1)):
        raise ValueError("scores rows must be equally spaced with a contiguous last axis")
    row_stride = scores.stride(1) if H > 1 else (scores.stride(0) if L > 1 else N)
    p = make_evict_params(L, H, N, budget, current, row_stride)
    if L * H > 0 and N > 0:
        last = (L * H - 1) * p.row_stride + N  # elements the library may read
        avail = scores.untyped_storage().nbytes() // 4 - scores.storage_offset()
        if last > avail:
            raise ValueError("scores view extends past its storage")
    own_keep = keep is None
    if own_keep:
        keep = torch.empty((L, H, N), dtype=torch.uint8, device=scores.device)
    elif keep.shape != (L, H, N) or keep.dtype != torch.uint8 or not keep.is_contiguous() \
            or keep.device != scores.device:
        raise ValueError("keep must be a contiguous uint8 [L, H, N] tensor on the scores' device")
    if kept_per_row is not None and (kept_per_row.shape != (L, H) or kept_per_row.dtype != torch.int32
                                     or not kept_per_row.is_contiguous()
                                     or kept_per_row.device != scores.device):
        raise ValueError("kept_per_row must be a contiguous int32 [L, H] tensor on the scores' device")
    need = kv_evict_workspace_size(p)
    own_workspace = bool(need) and workspace is None
    if own_workspace:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    elif workspace is not None and workspace.device != scores.device:
        raise ValueError("workspace must be on the scores' device")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.kv_evict_select(scores.data_ptr(), keep.data_ptr(),
                              kept_per_row.data_ptr() if kept_per_row is not None else None,
                              ctypes.byref(p), ws_ptr, ws_bytes, _stream_handle(stream))
    if st != KV_ATTN_OK:
        raise KvAttnError(st, "kv_evict_select")
    # Buffers allocated here on the current stream must outlive the launches on `stream`.
    if own_workspace:
        _hold_for_stream(workspace, stream)
    if own_keep:
        _hold_for_stream(keep, stream)
    return keep
