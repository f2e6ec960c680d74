"""paged_kv_cache_257_amd -- paged KV cache and PagedAttention decode on MI355X.

The product is the C-ABI library ``lib/libpkv.so`` (include/pkv.h): a C++
block allocator and HIP kernels for gfx950.  This package is its thin Python
binding: ``Pool`` mirrors the pkv_* calls, ``DecodeIteration`` strings them
into one decode iteration, ``PagedKVCache`` and ``attention`` give one
sequence the dense cache's append / read / reset surface.  Importing it does not load the library; the
first call does, and raises if it is not built (there is no fallback).
"""

from ._capi import PkvError, load  # noqa: F401
from .pool import (Pool, decode_plan, decode_plan_shared, decode_workspace_bound, decode_workspace_bytes,  # noqa: F401
                   default_partition_tokens, fill_partition, prefill_plan, prefill_workspace_bytes)

__all__ = ["Pool", "PkvError", "decode_plan", "decode_plan_shared", "decode_workspace_bound", "decode_workspace_bytes",
           "default_partition_tokens", "fill_partition", "prefill_plan", "prefill_workspace_bytes", "load",
           "DecodeIteration", "PagedKVCache", "attention"]


def __getattr__(name):
    if name == "DecodeIteration":
        from .step import DecodeIteration
        return DecodeIteration
    if name in ("PagedKVCache", "attention"):
        from . import cache
        return getattr(cache, name)
    raise AttributeError(name)
