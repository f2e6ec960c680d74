"""The dense cache's surface over the paged pool: ``PagedKVCache`` and
``attention``.

The preview page ("04 — Hacia PagedAttention", section "Lo que la Fase 22
construye hacia la Fase 27") asks that the paged cache replace the dense one
without its users noticing: the same append / read / reset, and an attention
call whose cache argument is optional.  Here one ``PagedKVCache`` is one
sequence of a shared ``Pool``.  Its methods string library calls together
(allocator, copy_blocks, write_kv, read_kv, the attention kernels) and move
the small host arrays they need to the device; nothing is computed in
Python.  This is the convenience surface, not the serving loop: every call
plans and allocates its own scratch on torch's current stream, where the
stepper and the pool calls reuse theirs.
"""

from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np
import torch

from .pool import (Pool, decode_plan, decode_workspace_bytes, prefill_plan,
                   prefill_workspace_bytes)

_DTYPE_NAMES = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


def _dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class PagedKVCache:
    """One sequence's K/V in a shared paged pool, behind append / read / reset.

    The sequence is created by the first append and released by ``reset``;
    ``fork`` gives a second cache sharing every block (the first divergent
    append copies the shared partly filled block).  Copy-on-write pairs are
    taken from the pool and copied before each write, so every append to the
    pool should go through a cache (or take its own pairs the same way)."""

    def __init__(self, pool: Pool):
        if pool.k_cache is None or pool.v_cache is None:
            raise ValueError("PagedKVCache needs a pool with device K/V arrays")
        self.pool = pool
        self.seq: Optional[int] = None

    def __len__(self) -> int:
        return 0 if self.seq is None else self.pool.length(self.seq)

    @property
    def device(self):
        return self.pool.k_cache.device

    def _check_rows(self, k, v, T: int) -> None:
        d = self.pool.desc
        shape = (T, d.num_kv_heads, d.head_dim)
        if tuple(k.shape) != shape or tuple(v.shape) != shape:
            raise ValueError(f"k and v must be shaped {shape}, got {tuple(k.shape)} and {tuple(v.shape)}")
        if k.dtype != self.pool.k_cache.dtype or v.dtype != self.pool.k_cache.dtype:
            raise ValueError("k and v must have the pool's dtype")

    def _take_slots(self, T: int) -> np.ndarray:
        """Allocator half of an append: slots of T new positions, copy-on-write done."""
        if self.seq is None:
            self.seq, slots = self.pool.alloc(T)
        else:
            slots = self.pool.append(self.seq, T)
        pairs = self.pool.take_cow()
        if len(pairs):
            self.pool.copy_blocks(_dev(pairs, self.device))
        return slots

    def append(self, k: torch.Tensor, v: torch.Tensor) -> np.ndarray:
        """Store T new tokens (k, v: device [T][H_kv][d] of the pool dtype)
        after the ones held; returns their slots."""
        T = int(k.shape[0])
        self._check_rows(k, v, T)
        if T == 0:
            return np.empty(0, dtype=np.int64)
        slots = self._take_slots(T)
        self.pool.write_kv(k.contiguous(), v.contiguous(), _dev(slots, self.device))
        return slots

    def read(self) -> Tuple[torch.Tensor, torch.Tensor]:
        """Dense K and V of every token held, device [L][H_kv][d] in
        position order, bit for bit what was appended."""
        d = self.pool.desc
        L = len(self)
        k = torch.empty((L, d.num_kv_heads, d.head_dim), dtype=self.pool.k_cache.dtype, device=self.device)
        v = torch.empty_like(k)
        if L:
            self.pool.read_kv(_dev(self.pool.slots(self.seq, 0, L), self.device), k, v)
        return k, v

    def reset(self) -> None:
        """Forget every token: the sequence's blocks go back to the pool."""
        if self.seq is not None:
            self.pool.free(self.seq)
            self.seq = None

    def fork(self) -> "PagedKVCache":
        child = PagedKVCache(self.pool)
        if self.seq is not None:
            child.seq = self.pool.fork(self.seq)
        return child

    def block_table(self) -> Tuple[np.ndarray, np.ndarray]:
        """(table [1][ceil(L/16)], lens [1]) of this sequence, host int32."""
        blocks = max(1, -(-len(self) // self.pool.desc.block_size))
        return self.pool.build_batch([self.seq], blocks)


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
              cache: Optional[PagedKVCache] = None, scale: Optional[float] = None) -> torch.Tensor:
    """Causal attention of T new tokens; returns fp32 [T][H_q][d].

    q: device [T][H_q][d]; k, v: device [T][H_kv][d]; one dtype (fp32, fp16
    or bf16); H_q a multiple of H_kv; scale defaults to 1/sqrt(d).

    With ``cache`` (holding L tokens), k and v are appended to it and query t
    sits at position L + t: it attends to the L cached tokens and the new
    ones up to itself.  One new token is a decode step (one launch stores
    its K/V and attends); more run the chunked-prefill kernel, or, for fp32
    pools (which that kernel does not take), one decode step per token.
    Without a cache the queries attend to the new tokens only, through a
    pool made for the call (paging does not change the result)."""
    if q.dim() != 3 or k.dim() != 3 or int(q.shape[0]) != int(k.shape[0]):
        raise ValueError("q must be [T][H_q][d] and k, v [T][H_kv][d] with the same T")
    T, Hq, D = (int(x) for x in q.shape)
    if cache is None:
        if q.dtype not in _DTYPE_NAMES:
            raise ValueError(f"unsupported dtype {q.dtype}")
        Hkv = int(k.shape[1])
        nb = max(1, -(-T // 16))
        kc = torch.zeros((nb, Hkv, 16, D), dtype=k.dtype, device=k.device)
        vc = torch.zeros_like(kc)
        pool = Pool(nb, Hkv, D, _DTYPE_NAMES[k.dtype], nb, 16, None, kc, vc)
        try:
            return attention(q, k, v, PagedKVCache(pool), scale)
        finally:
            pool.close()
    pool = cache.pool
    if D != pool.desc.head_dim or q.dtype != pool.k_cache.dtype:
        raise ValueError("q must have the pool's head_dim and dtype")
    cache._check_rows(k, v, T)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dev = cache.device
    out = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
    if T == 0:
        return out
    if T == 1:
        cache._take_slots(1)
        tables, lens = cache.block_table()
        plan, info = decode_plan(lens)
        ws_bytes = decode_workspace_bytes(info, Hq, D)
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
        pool.paged_decode(q.contiguous(), out, _dev(tables, dev), _dev(lens, dev), scale,
                          _dev(plan, dev), info, ws, k_new=k.contiguous(), v_new=v.contiguous())
        return out
    if pool.dtype == "f32":
        for t in range(T):
            out[t:t + 1] = attention(q[t:t + 1], k[t:t + 1], v[t:t + 1], cache, scale)
        return out
    cache.append(k, v)
    tables, lens = cache.block_table()
    plan, info = prefill_plan([T], lens, Hq, pool.desc.num_kv_heads, max_keys=-1)
    ws_bytes = prefill_workspace_bytes(info, D)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    pool.paged_prefill(q.contiguous(), out, _dev(tables, dev), _dev(lens, dev), scale,
                       _dev(plan, dev), info, ws)
    return out
