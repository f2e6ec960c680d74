"""Host mirrors of the paged K/V pools, and a dense shadow (oracle).

``MirrorPool`` holds K and V pools shaped ``[num_blocks][H_kv][block][d]``
in the storage dtype and zero-initialised, exactly the bits the device pools
should hold.  [preview] "La idea de PagedAttention" step 3 writes a new
token into its slot; slot s lives at block ``s // block`` and row
``s % block``.  A negative slot means "no write" (padding).  Copy-on-write
([lesson] paragraph 6) copies a whole block, K and V, every head.

``DenseShadow`` is the dense, never-paged cache of [preview] "Lo que funciona
en la Fase 22": per sequence, rows appended in logical order.  A fork copies
it.  The paged view gathered through a block table must equal it bit for
bit: paging changes where bytes live, not what is computed ([preview] "Lo que
deberías llevarte", item 2).

Reading: the pool layout is not on the pages; ``[block][head][row][d]`` keeps
each (block, head) tile contiguous.
"""

from __future__ import annotations

from typing import Dict, Sequence, Tuple

import numpy as np


class MirrorPool:
    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int,
                 storage_dtype, block_size: int = 16):
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        self.block_size = block_size
        self.k = np.zeros(shape, dtype=storage_dtype)
        self.v = np.zeros(shape, dtype=storage_dtype)

    def write_kv(self, k_new: np.ndarray, v_new: np.ndarray, slots: Sequence[int]) -> None:
        """Store token t's [H_kv][d] rows at slot ``slots[t]`` (skip negatives)."""
        slots = np.asarray(slots, dtype=np.int64)
        keep = slots >= 0
        s = slots[keep]
        assert len(np.unique(s)) == len(s), "slots of one write must be distinct"
        blk, row = s // self.block_size, s % self.block_size
        self.k[blk, :, row, :] = np.asarray(k_new)[keep]
        self.v[blk, :, row, :] = np.asarray(v_new)[keep]

    def copy_blocks(self, pairs: Sequence[Tuple[int, int]]) -> None:
        for src, dst in pairs:
            self.k[dst] = self.k[src]
            self.v[dst] = self.v[src]

    def gather(self, table: Sequence[int], length: int):
        """The sequence's logical K, V rows, each shaped [L][H_kv][d]."""
        if length == 0:
            H, d = self.k.shape[1], self.k.shape[3]
            e = np.zeros((0, H, d), self.k.dtype)
            return e, e.copy()
        t = np.asarray(table, dtype=np.int64)
        k = self.k[t].transpose(0, 2, 1, 3).reshape(-1, self.k.shape[1], self.k.shape[3])
        v = self.v[t].transpose(0, 2, 1, 3).reshape(-1, self.v.shape[1], self.v.shape[3])
        return k[:length], v[:length]


class DenseShadow:
    def __init__(self, num_kv_heads: int, head_dim: int, storage_dtype):
        self.H, self.d, self.dtype = num_kv_heads, head_dim, storage_dtype
        self.rows: Dict[int, Tuple[list, list]] = {}

    def new(self, seq: int) -> None:
        self.rows[seq] = ([], [])

    def append(self, seq: int, k_rows: np.ndarray, v_rows: np.ndarray) -> None:
        ks, vs = self.rows[seq]
        for t in range(len(k_rows)):
            ks.append(np.array(k_rows[t], copy=True))
            vs.append(np.array(v_rows[t], copy=True))

    def fork(self, parent: int, child: int) -> None:
        ks, vs = self.rows[parent]
        self.rows[child] = (list(ks), list(vs))

    def free(self, seq: int) -> None:
        del self.rows[seq]

    def get(self, seq: int):
        ks, vs = self.rows[seq]
        if not ks:
            e = np.zeros((0, self.H, self.d), self.dtype)
            return e, e.copy()
        return np.stack(ks), np.stack(vs)
