"""Split-KV decode attention for MI355X (gfx950).

The compute path is the C-ABI library ``libkvattn.so`` built from ``csrc/`` (hand-written HIP
kernels plus a small host layer). ``kv_cache_decode_split_amd.kv_attn`` is the thin ctypes
binding with the same function names as ``include/kv_attn.h``; importing it loads the library
and raises if it has not been built. ``workloads`` (seeded synthetic inputs) and
``accounting`` (bytes/FLOPs/roofline) are host-side helpers that never touch the data path.

Submodules are imported lazily so that the host-side helpers can be used on a machine where
the library is not built.
"""

import importlib

__all__ = ["kv_attn", "workloads", "accounting", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
