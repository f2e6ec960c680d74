"""Drive whole workloads through the oracle (test infrastructure only).

``DecodeRun``: a decode batch.  Sequence i (id i) is allocated with L_i
tokens from a pool whose free list starts in the seeded order; the context
K/V rows, drawn in sequence order, are written at the returned slots; each
sequence's query then attends over its L_i tokens.

``PrefillRun``: chunked prefill of a set of prompts.  Per step, for every
prompt with tokens left: allocate (first chunk) or append its next chunk's
tokens, write their K/V rows at the returned slots, then each chunk query
attends causally over the sequence as it now stands (gathered through the
block table).

``PrefixSharedRun``: the continuous-batching loop.  Per iteration, in
order: append one token to every live decoding sequence (ascending id) ->
copy-on-write copies, then the new K/V rows at their slots -> decode every
decoding sequence -> retire the seeded ``churn`` ids -> admit ``churn``
forks of seeded survivors.  The root prefix sequence (id 0) is never
decoded or retired.
"""

from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from workloads import STORAGE_NUMPY, draw_normal_storage
from workloads.churn import (STREAM_ITER_BASE, STREAM_PREFIX_K, STREAM_PREFIX_V,
                             STREAM_TAIL_K, STREAM_TAIL_V, choose_churn)

from .allocator import OracleAllocator
from .attention import decode_attention, prefill_attention, storage_to_f64
from .kvcache import MirrorPool


class DecodeRun:
    def __init__(self, cfg, lens, num_blocks, free_order, max_blocks_per_seq: int):
        self.cfg = cfg
        self.lens = [int(x) for x in lens]
        self.alloc = OracleAllocator(num_blocks, cfg.block_size, max_blocks_per_seq, free_order)
        self.mirror = MirrorPool(num_blocks, cfg.num_kv_heads, cfg.head_dim,
                                 STORAGE_NUMPY[cfg.dtype], cfg.block_size)
        self.seq_ids: List[int] = []
        slots: List[int] = []
        for L in self.lens:
            sid, s = self.alloc.alloc(L)
            self.seq_ids.append(sid)
            slots.extend(s)
        self.slots = np.asarray(slots, dtype=np.int64)

    def write_context(self, k_bits: np.ndarray, v_bits: np.ndarray) -> None:
        """k_bits, v_bits: [sum L][H_kv][d], rows in sequence order."""
        self.mirror.write_kv(k_bits, v_bits, self.slots)

    def tables(self, width: int):
        return self.alloc.build_batch(self.seq_ids, width)

    def attend(self, i: int, q_bits_i: np.ndarray) -> np.ndarray:
        """fp64 output [H_q][d] for batch entry i (gathered via its table)."""
        sid = self.seq_ids[i]
        K, V = self.mirror.gather(self.alloc.table(sid), self.alloc.length(sid))
        dt = self.cfg.dtype
        return decode_attention(storage_to_f64(q_bits_i, dt), storage_to_f64(K, dt),
                                storage_to_f64(V, dt), self.cfg.scale)


def iteration_values(cfg, t: int, n: int):
    """q [n][H_q][d], k, v [n][H_kv][d] storage bits drawn for iteration t."""
    dt = cfg.dtype
    q = draw_normal_storage((cfg.seed, STREAM_ITER_BASE + t, 1), (n, cfg.num_q_heads, cfg.head_dim), dt)
    k = draw_normal_storage((cfg.seed, STREAM_ITER_BASE + t, 2), (n, cfg.num_kv_heads, cfg.head_dim), dt)
    v = draw_normal_storage((cfg.seed, STREAM_ITER_BASE + t, 3), (n, cfg.num_kv_heads, cfg.head_dim), dt)
    return q, k, v


def prefix_values(cfg, tails: Sequence[int]):
    dt = cfg.dtype
    H, d = cfg.num_kv_heads, cfg.head_dim
    pk = draw_normal_storage((cfg.seed, STREAM_PREFIX_K), (cfg.prefix_len, H, d), dt)
    pv = draw_normal_storage((cfg.seed, STREAM_PREFIX_V), (cfg.prefix_len, H, d), dt)
    T = int(sum(int(t) for t in tails))
    tk = draw_normal_storage((cfg.seed, STREAM_TAIL_K), (T, H, d), dt)
    tv = draw_normal_storage((cfg.seed, STREAM_TAIL_V), (T, H, d), dt)
    return pk, pv, tk, tv


class PrefixSharedRun:
    def __init__(self, cfg, plan, max_blocks_per_seq: int, with_mirror: bool = True):
        self.cfg = cfg
        self.alloc = OracleAllocator(plan.num_blocks, cfg.block_size, max_blocks_per_seq,
                                     plan.free_order)
        self.mirror: Optional[MirrorPool] = None
        if with_mirror:
            self.mirror = MirrorPool(plan.num_blocks, cfg.num_kv_heads, cfg.head_dim,
                                     STORAGE_NUMPY[cfg.dtype], cfg.block_size)
        self.tails = [int(t) for t in plan.tails]

    def setup(self, values=None):
        """Root prefix, then every sequence forked from it with its own tail."""
        root, pslots = self.alloc.alloc(self.cfg.prefix_len)
        assert root == 0
        tail_slots: List[int] = []
        for t in self.tails:
            child = self.alloc.fork(root)
            tail_slots.extend(self.alloc.append(child, t))
        self.prefix_slots = np.asarray(pslots, dtype=np.int64)
        self.tail_slots = np.asarray(tail_slots, dtype=np.int64)
        if self.mirror is not None and values is not None:
            pk, pv, tk, tv = values
            self.mirror.write_kv(pk, pv, self.prefix_slots)
            self.mirror.write_kv(tk, tv, self.tail_slots)

    def decoding(self) -> List[int]:
        return [s for s in self.alloc.live() if s != 0]

    def append_step(self):
        """Append one token to each decoding sequence; returns (seqs, slots, cow)."""
        seqs = self.decoding()
        slots = [s[0] for s in self.alloc.append_batch(seqs, 1)]
        cow = self.alloc.take_cow()
        return seqs, np.asarray(slots, dtype=np.int64), cow

    def write_step(self, cow, k_bits, v_bits, slots) -> None:
        if self.mirror is not None:
            self.mirror.copy_blocks(cow)
            self.mirror.write_kv(k_bits, v_bits, slots)

    def churn_step(self, t: int):
        retire, parents = choose_churn(self.cfg, t, self.decoding())
        for s in retire:
            self.alloc.free_seq(s)
        children = [self.alloc.fork(p) for p in parents]
        return retire, parents, children

    def attend(self, seq: int, q_bits: np.ndarray) -> np.ndarray:
        K, V = self.mirror.gather(self.alloc.table(seq), self.alloc.length(seq))
        dt = self.cfg.dtype
        return decode_attention(storage_to_f64(q_bits, dt), storage_to_f64(K, dt),
                                storage_to_f64(V, dt), self.cfg.scale)


class PrefillRun:
    """Drives a ``workloads.prefill`` schedule through the oracle allocator
    and a mirrored pool."""

    def __init__(self, cfg, shapes, max_blocks_per_seq: int, values):
        from workloads.prefill import prompt_offsets
        self.cfg = cfg
        self.shapes = shapes
        self.alloc = OracleAllocator(shapes.num_blocks, cfg.block_size, max_blocks_per_seq,
                                     shapes.free_order)
        self.mirror = MirrorPool(shapes.num_blocks, cfg.num_kv_heads, cfg.head_dim,
                                 STORAGE_NUMPY[cfg.dtype], cfg.block_size)
        self.q, self.k, self.v = values
        self.row0 = prompt_offsets(shapes.prompts)
        self.step_index = 0

    def append_step(self):
        """Allocate / append the next chunk of every unfinished prompt and
        write its K/V rows.  Returns [(seq, first token, tokens, slots)]."""
        items = []
        for seq, t0, n in self.shapes.steps[self.step_index]:
            if t0 == 0:
                sid, slots = self.alloc.alloc(n)
                assert sid == seq
            else:
                slots = self.alloc.append(seq, n)
            slots = np.asarray(slots, dtype=np.int64)
            r = int(self.row0[seq]) + t0
            self.mirror.write_kv(self.k[r:r + n], self.v[r:r + n], slots)
            items.append((seq, t0, n, slots))
        self.step_index += 1
        return items

    def attend(self, seq: int, t0: int, n: int, rows=None) -> np.ndarray:
        """fp64 outputs [n][H_q][d] of chunk tokens t0 .. t0 + n - 1 of
        ``seq`` (the sequence must hold exactly t0 + n tokens).  ``rows``
        (optional) picks a subset of the chunk's tokens; the result then
        has len(rows) entries."""
        L = self.alloc.length(seq)
        assert L == t0 + n
        K, V = self.mirror.gather(self.alloc.table(seq), L)
        dt = self.cfg.dtype
        r = int(self.row0[seq]) + t0
        q = storage_to_f64(self.q[r:r + n], dt)
        K, V = storage_to_f64(K, dt), storage_to_f64(V, dt)
        if rows is None:
            return prefill_attention(q, K, V, self.cfg.scale)
        C = L - n
        return np.stack([decode_attention(q[t], K[:C + t + 1], V[:C + t + 1], self.cfg.scale)
                         for t in rows])
