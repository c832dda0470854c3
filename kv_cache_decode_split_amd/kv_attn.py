"""ctypes binding of ``libkvattn.so`` with the same names as ``include/kv_attn.h``.

Argument marshalling only: tensors are checked against the sizes the call implies (so that no
launch can address memory outside them), turned into raw device pointers, strides and sizes,
and handed to the C library together with torch's current HIP stream. Every step of the
attention runs in the library's HIP kernels; there is no fallback. Importing this module loads
the library and raises ImportError if it has not been built
(``python -m kv_cache_decode_split_amd.build``).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = [
    "LIB_PATH",
    "KvAttnError",
    "kv_attn_params",
    "kv_attn_plan",
    "make_params",
    "kv_attn_abi_version",
    "kv_attn_status_string",
    "kv_attn_get_plan",
    "kv_attn_workspace_size",
    "kv_attn_decode",
    "kv_attn_decode_split",
    "kv_attn_decode_merge",
    "kv_attn_decode_workload",
    "kv_attn_append",
    "kv_attn_append_decode",
    "DecodeCall",
    "decode_call_for",
    "kv_attn_merge",
    "kv_attn_validate_host",
    "kv_attn_scores_workspace_size",
    "kv_attn_decode_scores",
    "kv_attn_decode_noalloc",
    "kv_attn_read_probe",
    "KV_ATTN_PROBE_CHUNK",
    "KV_ATTN_NOALLOC_SCRATCH_BYTES",
    "EXPORTED_SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvattn.so")

KV_ATTN_OK = 0
KV_ATTN_ERR_NULL = 1
KV_ATTN_ERR_SHAPE = 2
KV_ATTN_ERR_UNSUPPORTED = 3
KV_ATTN_ERR_WORKSPACE = 4
KV_ATTN_ERR_HIP = 5
KV_ATTN_ERR_TABLE = 6
KV_ATTN_ERR_VALUE = 7
KV_ATTN_ERR_SCRATCH = 8

KV_ATTN_F32 = 0
KV_ATTN_BF16 = 1

EXPORTED_SYMBOLS = (
    "kv_attn_abi_version",
    "kv_attn_status_string",
    "kv_attn_get_plan",
    "kv_attn_workspace_size",
    "kv_attn_decode",
    "kv_attn_decode_split",
    "kv_attn_decode_merge",
    "kv_attn_append",
    "kv_attn_append_decode",
    "kv_attn_merge",
    "kv_attn_validate_host",
    "kv_attn_scores_workspace_size",
    "kv_attn_decode_scores",
    "kv_attn_decode_noalloc",
    "kv_attn_read_probe",
)

KV_ATTN_PROBE_CHUNK = 1 << 20
KV_ATTN_NOALLOC_SCRATCH_BYTES = 64 << 20


class KvAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        super().__init__(f"{where}: {kv_attn_status_string(status)} (status {status})")


class kv_attn_params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_ctx_len", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("window", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("k_stride_block", ctypes.c_int64),
        ("k_stride_token", ctypes.c_int64),
        ("k_stride_head", ctypes.c_int64),
        ("v_stride_block", ctypes.c_int64),
        ("v_stride_token", ctypes.c_int64),
        ("v_stride_head", ctypes.c_int64),
        ("num_sinks", ctypes.c_int32),
        ("num_queries", ctypes.c_int32),
    ]


class kv_attn_plan(ctypes.Structure):
    _fields_ = [
        ("num_splits", ctypes.c_int32),
        ("split_len", ctypes.c_int32),
        ("grid_split", ctypes.c_int32),
        ("grid_merge", ctypes.c_int32),
        ("kernel_variant", ctypes.c_int32),
        ("group_padded", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("wave_heads", ctypes.c_int32),
        ("unit_order", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_uint64),
        ("ml_offset", ctypes.c_uint64),
        ("order_offset", ctypes.c_uint64),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m kv_cache_decode_split_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    lib.kv_attn_abi_version.argtypes = []
    lib.kv_attn_abi_version.restype = ctypes.c_int32
    lib.kv_attn_status_string.argtypes = [ctypes.c_int32]
    lib.kv_attn_status_string.restype = ctypes.c_char_p
    lib.kv_attn_get_plan.argtypes = [P(kv_attn_params), ctypes.c_int32, P(kv_attn_plan)]
    lib.kv_attn_get_plan.restype = ctypes.c_int
    lib.kv_attn_workspace_size.argtypes = [P(kv_attn_params)]
    lib.kv_attn_workspace_size.restype = ctypes.c_size_t
    lib.kv_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, P(kv_attn_params), vp, ctypes.c_size_t, vp]
    lib.kv_attn_decode.restype = ctypes.c_int
    lib.kv_attn_decode_split.argtypes = [vp, vp, vp, vp, vp, vp, P(kv_attn_params), vp, ctypes.c_size_t, vp]
    lib.kv_attn_decode_split.restype = ctypes.c_int
    lib.kv_attn_decode_merge.argtypes = [vp, vp, P(kv_attn_params), vp, ctypes.c_size_t, vp]
    lib.kv_attn_decode_merge.restype = ctypes.c_int
    lib.kv_attn_append.argtypes = [vp, vp, vp, vp, vp, vp, P(kv_attn_params), vp]
    lib.kv_attn_append.restype = ctypes.c_int
    lib.kv_attn_append_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, P(kv_attn_params), vp,
                                          ctypes.c_size_t, vp]
    lib.kv_attn_append_decode.restype = ctypes.c_int
    lib.kv_attn_merge.argtypes = [vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp]
    lib.kv_attn_merge.restype = ctypes.c_int
    lib.kv_attn_validate_host.argtypes = [vp, vp, P(kv_attn_params)]
    lib.kv_attn_validate_host.restype = ctypes.c_int
    lib.kv_attn_scores_workspace_size.argtypes = [P(kv_attn_params)]
    lib.kv_attn_scores_workspace_size.restype = ctypes.c_size_t
    lib.kv_attn_decode_scores.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32,
                                          P(kv_attn_params), vp, ctypes.c_size_t, vp]
    lib.kv_attn_decode_scores.restype = ctypes.c_int
    lib.kv_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, P(kv_attn_params), vp]
    lib.kv_attn_decode_noalloc.restype = ctypes.c_int
    lib.kv_attn_read_probe.argtypes = [vp, ctypes.c_uint64, vp, vp]
    lib.kv_attn_read_probe.restype = ctypes.c_int
    return lib


_lib = _load()


def kv_attn_abi_version() -> int:
    return int(_lib.kv_attn_abi_version())


def kv_attn_status_string(status: int) -> str:
    return _lib.kv_attn_status_string(int(status)).decode()


def kv_attn_read_probe(src: torch.Tensor, sink: torch.Tensor) -> None:
    """Stream every byte of ``src`` (a contiguous CUDA tensor) once with the read probe, on the
    current stream; ``sink`` is a CUDA tensor with at least one 32-bit element."""
    if not (src.is_cuda and sink.is_cuda and src.is_contiguous()) or sink.device != src.device:
        raise ValueError("read probe: src and sink must be CUDA tensors on one device, src contiguous")
    _check_device(src, "src")
    if sink.numel() < 1 or sink.element_size() != 4:
        raise ValueError("read probe: sink must hold a 32-bit word")
    stream = torch.cuda.current_stream(src.device).cuda_stream
    st = _lib.kv_attn_read_probe(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(), stream)
    if st != KV_ATTN_OK:
        raise KvAttnError(st, "kv_attn_read_probe")


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return KV_ATTN_BF16
    if dt == torch.float32:
        return KV_ATTN_F32
    raise TypeError(f"unsupported dtype {dt} (float32 or bfloat16)")


def make_params(*, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                block_size: int, max_ctx_len: int, num_blocks: int,
                k_strides: Sequence[int], v_strides: Sequence[int],
                max_blocks_per_seq: int = 1, num_splits: int = 0,
                q_dtype: int = KV_ATTN_BF16, kv_dtype: int = KV_ATTN_BF16,
                scale: float = 0.0, window: Optional[int] = None,
                num_sinks: int = 0, num_queries: int = 1) -> kv_attn_params:
    """Fill a ``kv_attn_params`` (strides are (block, token, head) in elements).

    ``window=None`` attends every position; an integer W >= 1 attends the last W positions of
    each sequence plus its first ``num_sinks`` positions. ``num_queries`` (gamma) query tokens
    per sequence attend causally among themselves (the last gamma cached positions).
    """
    if window is not None and int(window) < 1:
        raise ValueError("window must be None (no window) or >= 1")
    p = kv_attn_params()
    p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim = batch, num_q_heads, num_kv_heads, head_dim
    p.block_size, p.max_blocks_per_seq, p.max_ctx_len = block_size, max_blocks_per_seq, max_ctx_len
    p.num_splits, p.q_dtype, p.kv_dtype, p.scale = num_splits, q_dtype, kv_dtype, scale
    p.window = 0 if window is None else int(window)
    p.num_sinks = int(num_sinks)
    p.num_queries = int(num_queries)
    p.num_blocks = num_blocks
    p.k_stride_block, p.k_stride_token, p.k_stride_head = (int(s) for s in k_strides)
    p.v_stride_block, p.v_stride_token, p.v_stride_head = (int(s) for s in v_strides)
    return p


def kv_attn_get_plan(params: kv_attn_params, num_cus: int = 0) -> dict:
    plan = kv_attn_plan()
    st = _lib.kv_attn_get_plan(ctypes.byref(params), int(num_cus), ctypes.byref(plan))
    if st != KV_ATTN_OK:
        raise KvAttnError(st, "kv_attn_get_plan")
    return {name: getattr(plan, name) for name, _ in kv_attn_plan._fields_}


def kv_attn_workspace_size(params: kv_attn_params) -> int:
    return int(_lib.kv_attn_workspace_size(ctypes.byref(params)))


def kv_attn_validate_host(block_table, ctx_lens, params: kv_attn_params) -> int:
    """Host-side content check; ``block_table``/``ctx_lens`` are CPU int32 tensors (or None)."""
    ctx = ctx_lens.detach().to("cpu", torch.int32).contiguous()
    bt = None if block_table is None else block_table.detach().to("cpu", torch.int32).contiguous()
    return int(_lib.kv_attn_validate_host(None if bt is None else bt.data_ptr(), ctx.data_ptr(),
                                          ctypes.byref(params)))


def _stream_handle(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _hold_for_stream(t: Optional[torch.Tensor], stream) -> None:
    """Keep torch's caching allocator from reusing ``t`` (allocated here, on the current stream)
    while the kernels just enqueued on ``stream`` may still use it: when ``stream`` is another
    stream, the block is released only once that stream's work has passed this point."""
    if t is not None and stream is not None and stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)


def _check_device(t: torch.Tensor, what: str) -> None:
    """The library takes device pointers and launches on the current device: a host tensor, or
    one on another device, is refused here rather than handed to a kernel."""
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device (CUDA) tensor, not on {t.device}")
    current = torch.cuda.current_device()
    if t.device.index != current:
        raise ValueError(f"{what} is on {t.device} but the library launches on the current device "
                         f"cuda:{current}")


def _check_extent(t: torch.Tensor, strides, blocks: int, slots: int, heads: int, d: int, what: str):
    last = (blocks - 1) * strides[0] + (slots - 1) * strides[1] + (heads - 1) * strides[2] + d - 1
    avail = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
    if last >= avail:
        raise ValueError(f"{what}: strides address element {last} but only {avail} exist")


class DecodeCall:
    """Checked, marshalled arguments of one decode problem (reusable across launches).

    q: [B, h_q, d] (one query token per sequence) or [B, gamma, h_q, d] (gamma tokens, the last
    gamma cached positions, causal among themselves), contiguous bf16/fp32; out: fp32 shaped
    like q. k_cache/v_cache:
    device tensors of one dtype holding num_kv_heads heads, whose element (block, token, head, i)
    is at block*strides[0] + token*strides[1] + head*strides[2] + i. block_table: int32
    [B, max_blocks] (paged; block_size tokens per block) or None (contiguous; block_size = slot
    capacity). ctx_lens: int32 [B] on the device. max_ctx_len defaults to ctx_lens.max() (a host
    sync). The workspace, if not given, is allocated once from torch's allocator. ``window`` /
    ``num_sinks`` restrict attention to the first num_sinks and last window positions.
    """

    def __init__(self, q, k_cache, v_cache, block_table, ctx_lens, out, *, num_kv_heads: int,
                 k_strides: Sequence[int], v_strides: Sequence[int], block_size: int,
                 num_blocks: int, max_ctx_len: Optional[int] = None, scale: float = 0.0,
                 num_splits: int = 0, workspace: Optional[torch.Tensor] = None,
                 window: Optional[int] = None, num_sinks: int = 0, with_scores: bool = False,
                 allocate_workspace: bool = True):
        if q.dim() not in (3, 4) or not q.is_contiguous():
            raise ValueError("q must be a contiguous [B, h_q, d] or [B, gamma, h_q, d] tensor")
        B, hq, d = q.shape[0], q.shape[-2], q.shape[-1]
        nq = int(q.shape[1]) if q.dim() == 4 else 1
        self.num_queries = nq
        if out.shape != q.shape or out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError("out must be a contiguous fp32 tensor shaped like q")
        if k_cache.dtype != v_cache.dtype:
            raise ValueError("k_cache and v_cache must share a dtype")
        dev = q.device
        _check_device(q, "q")
        for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("ctx_lens", ctx_lens),
                        ("out", out)):
            if t.device != dev:
                raise ValueError(f"{name} is on {t.device}, q on {dev}")
        if ctx_lens.dtype != torch.int32 or ctx_lens.shape != (B,) or not ctx_lens.is_contiguous():
            raise ValueError("ctx_lens must be a contiguous int32 [B] tensor")
        if block_table is not None:
            if (block_table.dtype != torch.int32 or block_table.dim() != 2
                    or block_table.shape[0] != B or not block_table.is_contiguous()
                    or block_table.device != dev):
                raise ValueError("block_table must be a contiguous int32 [B, max_blocks] device tensor")
            max_blocks = int(block_table.shape[1])
        else:
            max_blocks = 1
        if max_ctx_len is None:
            max_ctx_len = int(ctx_lens.max().item()) if B else 0
        hkv = int(num_kv_heads)
        self.params = make_params(
            batch=B, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=block_size,
            max_ctx_len=int(max_ctx_len), num_blocks=num_blocks, k_strides=k_strides,
            v_strides=v_strides, max_blocks_per_seq=max_blocks, num_splits=num_splits,
            q_dtype=_dtype_code(q.dtype), kv_dtype=_dtype_code(k_cache.dtype), scale=float(scale),
            window=window, num_sinks=num_sinks, num_queries=nq)
        _check_extent(k_cache, k_strides, num_blocks, block_size, hkv, d, "k_cache")
        _check_extent(v_cache, v_strides, num_blocks, block_size, hkv, d, "v_cache")
        ws_bytes = (kv_attn_scores_workspace_size(self.params) if with_scores
                    else kv_attn_workspace_size(self.params))
        if with_scores and ws_bytes == 0:
            raise KvAttnError(KV_ATTN_ERR_UNSUPPORTED, "kv_attn_scores_workspace_size")
        # A workspace allocated here belongs to this call; one the caller passes is the caller's
        # (who then keeps it alive until the launches that use it have finished).
        self._own_workspace = bool(ws_bytes) and workspace is None and allocate_workspace
        if self._own_workspace:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        if workspace is not None and workspace.device != dev:
            raise ValueError("workspace must be on q's device")
        self.workspace = workspace
        self._keep = (q, k_cache, v_cache, block_table, ctx_lens, out)
        self._ptrs = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                      None if block_table is None else block_table.data_ptr(),
                      ctx_lens.data_ptr(), out.data_ptr())
        self._ws = (workspace.data_ptr() if workspace is not None else None,
                    workspace.numel() * workspace.element_size() if workspace is not None else 0)

    def plan(self) -> dict:
        return kv_attn_get_plan(self.params)

    def _launched_on(self, stream) -> None:
        if self._own_workspace:
            _hold_for_stream(self.workspace, stream)

    def decode(self, stream=None) -> None:
        st = _lib.kv_attn_decode(*self._ptrs, ctypes.byref(self.params), *self._ws,
                                 _stream_handle(stream))
        if st != KV_ATTN_OK:
            raise KvAttnError(st, "kv_attn_decode")
        self._launched_on(stream)

    def decode_noalloc(self, stream=None) -> None:
        """kv_attn_decode_noalloc: the split states go to the library's own device scratch
        (nothing is allocated; calls that overlap on one device race on that scratch)."""
        st = _lib.kv_attn_decode_noalloc(*self._ptrs, ctypes.byref(self.params),
                                         _stream_handle(stream))
        if st != KV_ATTN_OK:
            raise KvAttnError(st, "kv_attn_decode_noalloc")

    def decode_scores(self, token_scores: torch.Tensor, accumulate: bool = False,
                      stream=None) -> None:
        """Decode and write (or, with ``accumulate``, add) each attended position's attention
        weight summed over its KV head's query heads into ``token_scores``, a contiguous fp32
        [B, h_kv, max_ctx_len] tensor (build the call with ``with_scores=True``)."""
        p = self.params
        want = (p.batch, p.num_kv_heads, p.max_ctx_len)
        if (tuple(token_scores.shape) != want or token_scores.dtype != torch.float32
                or not token_scores.is_contiguous() or token_scores.device != self._keep[0].device):
            raise ValueError(f"token_scores must be a contiguous fp32 {list(want)} tensor on q's device")
        st = _lib.kv_attn_decode_scores(*self._ptrs, token_scores.data_ptr(), int(bool(accumulate)),
                                        ctypes.byref(self.params), *self._ws, _stream_handle(stream))
        if st != KV_ATTN_OK:
            raise KvAttnError(st, "kv_attn_decode_scores")
        self._launched_on(stream)

    def split(self, stream=None) -> None:
        st = _lib.kv_attn_decode_split(*self._ptrs, ctypes.byref(self.params), *self._ws,
                                       _stream_handle(stream))
        if st != KV_ATTN_OK:
            raise KvAttnError(st, "kv_attn_decode_split")
        self._launched_on(stream)

    def merge(self, stream=None) -> None:
        st = _lib.kv_attn_decode_merge(self._ptrs[4], self._ptrs[5], ctypes.byref(self.params),
                                       *self._ws, _stream_handle(stream))
        if st != KV_ATTN_OK:
            raise KvAttnError(st, "kv_attn_decode_merge")
        self._launched_on(stream)

    def append_decode(self, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
        """Write each sequence's new K/V rows at positions ctx_lens[b] - gamma .. ctx_lens[b] - 1
        (k_new/v_new [B, h_kv, d] for gamma = 1, else [B, gamma, h_kv, d]), then decode."""
        q, k_cache = self._keep[0], self._keep[1]
        _check_new_rows(k_new, v_new, k_cache, q.shape[0], self.params.num_kv_heads, q.shape[-1],
                        self.num_queries)
        st = _lib.kv_attn_append_decode(self._ptrs[0], k_new.data_ptr(), v_new.data_ptr(),
                                        *self._ptrs[1:], ctypes.byref(self.params), *self._ws,
                                        _stream_handle(stream))
        if st != KV_ATTN_OK:
            raise KvAttnError(st, "kv_attn_append_decode")
        self._launched_on(stream)


def _check_new_rows(k_new, v_new, cache, batch, num_kv_heads, head_dim, rows=1):
    want = (batch, num_kv_heads, head_dim) if rows == 1 else (batch, rows, num_kv_heads, head_dim)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if (tuple(t.shape) != want or not t.is_contiguous()
                or t.dtype != cache.dtype or t.device != cache.device):
            raise ValueError(f"{name} must be a contiguous {list(want)} tensor of the cache's "
                             "dtype on its device")


def kv_attn_decode(q, k_cache, v_cache, block_table, ctx_lens, out, *, stream=None, **kwargs) -> None:
    """Enqueue one decode-attention step (both passes); arguments as for :class:`DecodeCall`."""
    DecodeCall(q, k_cache, v_cache, block_table, ctx_lens, out, **kwargs).decode(stream)


def kv_attn_decode_noalloc(q, k_cache, v_cache, block_table, ctx_lens, out, *, stream=None,
                           **kwargs) -> None:
    """One decode step with no device allocation at all (the library's fixed scratch holds the
    split states); arguments as for :class:`DecodeCall` (no workspace)."""
    DecodeCall(q, k_cache, v_cache, block_table, ctx_lens, out, allocate_workspace=False,
               **kwargs).decode_noalloc(stream)


def kv_attn_scores_workspace_size(params: kv_attn_params) -> int:
    return int(_lib.kv_attn_scores_workspace_size(ctypes.byref(params)))


def kv_attn_decode_scores(q, k_cache, v_cache, block_table, ctx_lens, out, token_scores, *,
                          accumulate: bool = False, stream=None, **kwargs) -> None:
    """Decode plus per-position attention weights (see :meth:`DecodeCall.decode_scores`)."""
    DecodeCall(q, k_cache, v_cache, block_table, ctx_lens, out, with_scores=True,
               **kwargs).decode_scores(token_scores, accumulate, stream)


def kv_attn_decode_split(q, k_cache, v_cache, block_table, ctx_lens, out, *, stream=None,
                         **kwargs) -> DecodeCall:
    """Enqueue the streaming pass only; returns the call (its workspace holds the split states)."""
    call = DecodeCall(q, k_cache, v_cache, block_table, ctx_lens, out, **kwargs)
    call.split(stream)
    return call


def kv_attn_decode_merge(call: DecodeCall, stream=None) -> None:
    """Enqueue the merge pass over the workspace of a :func:`kv_attn_decode_split` call."""
    call.merge(stream)


def kv_attn_append(k_new, v_new, k_cache, v_cache, block_table, positions, *, num_kv_heads: int,
                   k_strides: Sequence[int], v_strides: Sequence[int], block_size: int,
                   num_blocks: int, stream=None) -> None:
    """Store k_new/v_new ([B, h_kv, d]) at logical position positions[b] of every sequence, or
    ([B, n, h_kv, d]) n tokens at positions[b] .. positions[b] + n - 1."""
    B = int(positions.shape[0])
    d = int(k_new.shape[-1])
    n = int(k_new.shape[1]) if k_new.dim() == 4 else 1
    _check_device(k_cache, "k_cache")
    if v_cache.device != k_cache.device or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must share k_cache's device and dtype")
    _check_new_rows(k_new, v_new, k_cache, B, num_kv_heads, d, n)
    if positions.dtype != torch.int32 or not positions.is_contiguous() or positions.device != k_cache.device:
        raise ValueError("positions must be a contiguous int32 [B] tensor on the cache's device")
    if block_table is not None:
        if (block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B
                or not block_table.is_contiguous() or block_table.device != k_cache.device):
            raise ValueError("block_table must be a contiguous int32 [B, max_blocks] device tensor")
        max_blocks = int(block_table.shape[1])
    else:
        max_blocks = 1
    p = make_params(batch=B, num_q_heads=num_kv_heads, num_kv_heads=num_kv_heads, head_dim=d,
                    block_size=block_size, max_ctx_len=0, num_blocks=num_blocks, k_strides=k_strides,
                    v_strides=v_strides, max_blocks_per_seq=max_blocks,
                    kv_dtype=_dtype_code(k_cache.dtype), q_dtype=_dtype_code(k_cache.dtype),
                    num_queries=n)
    _check_extent(k_cache, k_strides, num_blocks, block_size, num_kv_heads, d, "k_cache")
    _check_extent(v_cache, v_strides, num_blocks, block_size, num_kv_heads, d, "v_cache")
    st = _lib.kv_attn_append(k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
                             v_cache.data_ptr(), None if block_table is None else block_table.data_ptr(),
                             positions.data_ptr(), ctypes.byref(p), _stream_handle(stream))
    if st != KV_ATTN_OK:
        raise KvAttnError(st, "kv_attn_append")


def kv_attn_append_decode(q, k_new, v_new, k_cache, v_cache, block_table, ctx_lens, out, *,
                          stream=None, **kwargs) -> None:
    """Append each sequence's new K/V at ctx_lens[b] - 1, then decode (one call, same stream)."""
    DecodeCall(q, k_cache, v_cache, block_table, ctx_lens, out, **kwargs).append_decode(
        k_new, v_new, stream)


def _workload_args(w) -> dict:
    ks, vs = w.kv_strides()
    args = dict(num_kv_heads=w.spec.num_kv_heads, k_strides=ks, v_strides=vs,
                block_size=w.block_size, num_blocks=w.num_blocks, max_ctx_len=w.max_ctx_len)
    if getattr(w.spec, "window", None) is not None:
        args.update(window=w.spec.window, num_sinks=w.spec.num_sinks)
    return args


def kv_attn_decode_workload(w, out: torch.Tensor, *, stream=None, **kwargs) -> None:
    """kv_attn_decode on a workload object (attributes q, k_cache, v_cache, block_table, ctx_lens,
    block_size, num_blocks, max_ctx_len, spec.num_kv_heads and kv_strides()), e.g. one built by
    ``kv_cache_decode_split_amd.workloads.make_workload``."""
    args = _workload_args(w)
    args.update(kwargs)
    kv_attn_decode(w.q, w.k_cache, w.v_cache, w.block_table, w.ctx_lens, out, stream=stream, **args)


def decode_call_for(w, out: torch.Tensor, **kwargs) -> DecodeCall:
    """A reusable :class:`DecodeCall` for a workload object."""
    args = _workload_args(w)
    args.update(kwargs)
    return DecodeCall(w.q, w.k_cache, w.v_cache, w.block_table, w.ctx_lens, out, **args)


def kv_attn_merge(o_partial: torch.Tensor, ml_partial: torch.Tensor,
                  num_valid: Optional[torch.Tensor], out: torch.Tensor, stream=None) -> None:
    """Merge split states: o_partial [rows, S, d], ml_partial [rows, S, 2] (base-2 maxima, sums),
    num_valid int32 [rows] or None, out [rows, d] fp32. All contiguous fp32 on one device."""
    if o_partial.dim() != 3 or ml_partial.dim() != 3:
        raise ValueError("o_partial must be [rows, S, d] and ml_partial [rows, S, 2]")
    rows, S, d = o_partial.shape
    _check_device(o_partial, "o_partial")
    if ml_partial.shape != (rows, S, 2) or out.shape != (rows, d):
        raise ValueError("shape mismatch between o_partial, ml_partial and out")
    for t in (o_partial, ml_partial, out):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.device != o_partial.device:
            raise ValueError("merge tensors must be contiguous fp32 on one device")
    if num_valid is not None and (num_valid.dtype != torch.int32 or num_valid.shape != (rows,)
                                  or not num_valid.is_contiguous()
                                  or num_valid.device != o_partial.device):
        raise ValueError("num_valid must be a contiguous int32 [rows] tensor on the same device")
    st = _lib.kv_attn_merge(o_partial.data_ptr(), ml_partial.data_ptr(),
                            None if num_valid is None else num_valid.data_ptr(), out.data_ptr(),
                            rows, S, d, _stream_handle(stream))
    if st != KV_ATTN_OK:
        raise KvAttnError(st, "kv_attn_merge")
