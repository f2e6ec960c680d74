"""Python face of libpkv: the same calls as include/pkv.h, marshalled.

Device memory and streams come from PyTorch; every computation runs in the
library (host allocator in C++, kernels in HIP).  Host arrays are numpy.
"""

from __future__ import annotations

import ctypes as C
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import _capi
from ._capi import PROBE_MODES, PlanInfo, PoolDesc, PrefillPlanInfo, Stats, check, i32p, i64p


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


class Pool:
    """A paged K/V pool: host allocator state plus (optionally) device K/V.

    ``k_cache`` / ``v_cache``: device tensors shaped
    [num_blocks][num_kv_heads][block_size][head_dim] of the pool dtype, or
    None for an allocator-only pool (``host_only=True`` loads the g++-built
    allocator library, usable without a GPU).
    """

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str,
                 max_blocks_per_seq: int, block_size: int = 16, free_order=None,
                 k_cache=None, v_cache=None, host_only: bool = False):
        self.lib = _capi.load(host_only=host_only)
        self.desc = PoolDesc(num_blocks, block_size, num_kv_heads, head_dim, max_blocks_per_seq,
                             _capi.DTYPES[dtype])
        self.dtype = dtype
        self.k_cache, self.v_cache = k_cache, v_cache
        order = None if free_order is None else np.ascontiguousarray(free_order, dtype=np.int32)
        h = C.c_void_p()
        check(self.lib, self.lib.pkv_pool_create(C.byref(self.desc), _dptr(k_cache), _dptr(v_cache),
                                                 i32p(order), C.byref(h)))
        self.handle = h

    def close(self):
        if self.handle:
            self.lib.pkv_pool_destroy(self.handle)
            self.handle = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 -- interpreter shutdown
            pass

    # ---- allocator -----------------------------------------------------------
    def reset(self):
        check(self.lib, self.lib.pkv_pool_reset(self.handle))

    def alloc(self, n_tokens: int) -> Tuple[int, np.ndarray]:
        sid = C.c_int32()
        slots = np.empty(max(n_tokens, 1), dtype=np.int64)
        check(self.lib, self.lib.pkv_seq_alloc(self.handle, n_tokens, C.byref(sid), i64p(slots)))
        return sid.value, slots[:n_tokens]

    def append(self, seq: int, n_tokens: int = 1) -> np.ndarray:
        slots = np.empty(max(n_tokens, 1), dtype=np.int64)
        check(self.lib, self.lib.pkv_seq_append(self.handle, seq, n_tokens, i64p(slots)))
        return slots[:n_tokens]

    def append_batch(self, seqs: Sequence[int], n_tokens: int = 1) -> np.ndarray:
        s = np.ascontiguousarray(seqs, dtype=np.int32)
        slots = np.empty((max(len(s), 1), max(n_tokens, 1)), dtype=np.int64)
        check(self.lib, self.lib.pkv_seq_append_batch(self.handle, i32p(s), len(s), n_tokens,
                                                      i64p(slots)))
        return slots[:len(s), :n_tokens]

    def fork(self, parent: int) -> int:
        c = C.c_int32()
        check(self.lib, self.lib.pkv_seq_fork(self.handle, parent, C.byref(c)))
        return c.value

    def fork_prefix(self, parent: int, n_tokens: int) -> int:
        c = C.c_int32()
        check(self.lib, self.lib.pkv_seq_fork_prefix(self.handle, parent, n_tokens, C.byref(c)))
        return c.value

    def free(self, seq: int) -> None:
        check(self.lib, self.lib.pkv_seq_free(self.handle, seq))

    def free_batch(self, seqs: Sequence[int]) -> None:
        arr = np.ascontiguousarray(seqs, dtype=np.int32)
        check(self.lib, self.lib.pkv_seq_free_batch(self.handle, i32p(arr), len(arr)))

    def fork_batch(self, parents: Sequence[int]) -> np.ndarray:
        arr = np.ascontiguousarray(parents, dtype=np.int32)
        kids = np.empty(len(arr), dtype=np.int32)
        check(self.lib, self.lib.pkv_seq_fork_batch(self.handle, i32p(arr), len(arr), i32p(kids)))
        return kids

    def length(self, seq: int) -> int:
        n = C.c_int32()
        check(self.lib, self.lib.pkv_seq_length(self.handle, seq, C.byref(n)))
        return n.value

    def table(self, seq: int) -> List[int]:
        cap = self.desc.max_blocks_per_seq
        buf = np.empty(cap, dtype=np.int32)
        n = C.c_int32()
        check(self.lib, self.lib.pkv_seq_table(self.handle, seq, i32p(buf), cap, C.byref(n)))
        return buf[:n.value].tolist()

    def slots(self, seq: int, first: int = 0, n: Optional[int] = None) -> np.ndarray:
        """int64 slots of positions [first, first + n) (n defaults to the rest)."""
        if n is None:
            n = self.length(seq) - first
        buf = np.empty(max(n, 1), dtype=np.int64)
        check(self.lib, self.lib.pkv_seq_slots(self.handle, seq, first, n, i64p(buf)))
        return buf[:n]

    def live(self) -> List[int]:
        n = C.c_int32()
        self.lib.pkv_live_seqs(self.handle, None, 0, C.byref(n))
        buf = np.empty(max(n.value, 1), dtype=np.int32)
        check(self.lib, self.lib.pkv_live_seqs(self.handle, i32p(buf), len(buf), C.byref(n)))
        return buf[:n.value].tolist()

    def free_list(self) -> List[int]:
        buf = np.empty(max(self.desc.num_blocks, 1), dtype=np.int32)
        n = C.c_int32()
        check(self.lib, self.lib.pkv_free_list(self.handle, i32p(buf), len(buf), C.byref(n)))
        return buf[:n.value].tolist()

    def refcounts(self) -> List[int]:
        buf = np.empty(max(self.desc.num_blocks, 1), dtype=np.int32)
        check(self.lib, self.lib.pkv_refcounts(self.handle, i32p(buf)))
        return buf[:self.desc.num_blocks].tolist()

    def stats(self) -> dict:
        s = Stats()
        check(self.lib, self.lib.pkv_stats(self.handle, C.byref(s)))
        return s.as_dict()

    def take_cow(self) -> np.ndarray:
        n = C.c_int32()
        self.lib.pkv_take_cow(self.handle, None, 0, C.byref(n))
        buf = np.empty((max(n.value, 1), 2), dtype=np.int32)
        check(self.lib, self.lib.pkv_take_cow(self.handle, i32p(buf), len(buf), C.byref(n)))
        return buf[:n.value]

    def build_batch(self, seqs: Sequence[int], table_stride: int,
                    tables: Optional[np.ndarray] = None, lens: Optional[np.ndarray] = None):
        s = np.ascontiguousarray(seqs, dtype=np.int32)
        if tables is None:
            tables = np.empty((len(s), table_stride), dtype=np.int32)
        if lens is None:
            lens = np.empty(len(s), dtype=np.int32)
        check(self.lib, self.lib.pkv_build_batch(self.handle, i32p(s), len(s), i32p(tables),
                                                 table_stride, i32p(lens)))
        return tables, lens

    # ---- device ----------------------------------------------------------------
    def write_kv(self, k_new, v_new, slot_mapping, stream=None) -> None:
        """k_new, v_new: device [T][H_kv][d]; slot_mapping: device int64 [T]."""
        n = int(slot_mapping.shape[0])
        check(self.lib, self.lib.pkv_write_kv(self.handle, _dptr(k_new), _dptr(v_new),
                                              _dptr(slot_mapping), n, _stream_ptr(stream)))

    def read_kv(self, slot_mapping, k_out, v_out, stream=None) -> None:
        """k_out, v_out: device [T][H_kv][d] filled from the pool rows at slot_mapping (int64 [T])."""
        n = int(slot_mapping.shape[0])
        check(self.lib, self.lib.pkv_read_kv(self.handle, _dptr(slot_mapping), n, _dptr(k_out),
                                             _dptr(v_out), _stream_ptr(stream)))

    def copy_blocks(self, pairs, stream=None) -> None:
        """pairs: device int32 [n][2] (src, dst)."""
        n = int(pairs.shape[0])
        check(self.lib, self.lib.pkv_copy_blocks(self.handle, _dptr(pairs), n, _stream_ptr(stream)))

    def batch_shared_kv(self, seqs) -> int:
        """The decode plan's load-policy hint for these sequences: 1 when a
        quarter or more of their context sits in blocks several sequences
        hold (set PlanInfo.shared_kv from it), else 0."""
        arr = np.ascontiguousarray(seqs, dtype=np.int32)
        out = C.c_int32()
        check(self.lib, self.lib.pkv_batch_shared_kv(self.handle, i32p(arr), len(arr), C.byref(out)))
        return out.value

    def decode_occupancy(self, num_q_heads: int) -> Tuple[int, int]:
        """(workgroups per decode work item, resident workgroups on the device)."""
        wpi, res = C.c_int32(), C.c_int64()
        check(self.lib, self.lib.pkv_decode_occupancy(self.handle, num_q_heads, C.byref(wpi), C.byref(res)))
        return wpi.value, res.value

    def paged_decode(self, q, out, block_tables, context_lens, scale: float, plan, info: PlanInfo,
                     workspace, stream=None, k_new=None, v_new=None, split: bool = False) -> None:
        """Decode attention of every sequence of the batch through its table.

        ``k_new``/``v_new`` (device [B][H_kv][d]) are the newest token's rows:
        stored into the pool and attended in the same launch.  ``workspace``
        must be zeroed before its first use.  ``split`` runs the two-launch
        variant (partition kernel, then the separate combine kernel)."""
        B, Hq = int(q.shape[0]), int(q.shape[1])
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        args = (self.handle, _dptr(q), _dptr(k_new), _dptr(v_new), _dptr(out), B, Hq,
                _dptr(block_tables), int(block_tables.shape[1]), _dptr(context_lens), float(scale),
                _dptr(plan), C.byref(info), _dptr(workspace), ws_bytes, _stream_ptr(stream))
        if split:
            check(self.lib, self.lib.pkv_paged_decode_partitions(*args))
            check(self.lib, self.lib.pkv_paged_decode_reduce(*args))
        else:
            check(self.lib, self.lib.pkv_paged_decode(*args))

    def paged_decode_noalloc(self, q, out, block_tables, context_lens, scale: float, plan, info: PlanInfo,
                             stream=None, k_new=None, v_new=None) -> None:
        """``paged_decode`` without a workspace: the library's fixed per-GPU
        scratch holds the split-K records (see pkv_paged_decode_noalloc)."""
        B, Hq = int(q.shape[0]), int(q.shape[1])
        check(self.lib, self.lib.pkv_paged_decode_noalloc(
            self.handle, _dptr(q), _dptr(k_new), _dptr(v_new), _dptr(out), B, Hq,
            _dptr(block_tables), int(block_tables.shape[1]), _dptr(context_lens), float(scale),
            _dptr(plan), C.byref(info), _stream_ptr(stream)))


    def gather_probe(self, block_tables, context_lens, plan, info: PlanInfo, out, mode: str = "regs",
                     waves: int = 4, lds_pad: int = 0, stream=None) -> None:
        """Read every K/V tile a decode of this plan reads, without its
        arithmetic (a measurement aid; see pkv_gather_probe).  ``out``: device
        uint32 tensor of at least n_work x num_kv_heads x waves entries."""
        check(self.lib, self.lib.pkv_gather_probe(
            self.handle, _dptr(block_tables), int(block_tables.shape[1]), _dptr(context_lens),
            int(info.num_seqs), _dptr(plan), C.byref(info), PROBE_MODES[mode], int(waves), int(lds_pad), _dptr(out),
            _stream_ptr(stream)))

    def paged_prefill(self, q, out, block_tables, context_lens, scale: float, plan,
                      info: PrefillPlanInfo, workspace=None, stream=None) -> None:
        """Causal attention of chunked-prefill queries (see pkv_paged_prefill).

        q: device [total_q][H_q][d] (pool dtype); out: device fp32, same
        shape; ``plan``/``info`` from ``prefill_plan`` (plan on the device);
        ``workspace``: zeroed device tensor of ``prefill_workspace_bytes``
        bytes when the plan splits tiles."""
        Hq = int(q.shape[1])
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        check(self.lib, self.lib.pkv_paged_prefill(
            self.handle, _dptr(q), _dptr(out), int(info.num_seqs), Hq, _dptr(block_tables),
            int(block_tables.shape[1]), _dptr(context_lens), float(scale), _dptr(plan),
            C.byref(info), _dptr(workspace), ws_bytes, _stream_ptr(stream)))


def prefill_plan(q_lens, context_lens, num_q_heads: int, num_kv_heads: int, max_keys: int = 0,
                 host_only: bool = False) -> Tuple[np.ndarray, PrefillPlanInfo]:
    """Host work list of a chunked-prefill launch (see pkv_prefill_plan);
    tiles attending more than ``max_keys`` keys (> 0) are split."""
    lib = _capi.load(host_only=host_only)
    ql = np.ascontiguousarray(q_lens, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    n = C.c_int32()
    check(lib, lib.pkv_prefill_plan_ints(i32p(ql), i32p(cl), len(ql), num_q_heads, num_kv_heads,
                                         int(max_keys), C.byref(n)))
    plan = np.empty(max(n.value, 1), dtype=np.int32)
    info = PrefillPlanInfo()
    check(lib, lib.pkv_prefill_plan(i32p(ql), i32p(cl), len(ql), num_q_heads, num_kv_heads,
                                    int(max_keys), i32p(plan), len(plan), C.byref(info)))
    return plan[:info.plan_ints], info


def prefill_workspace_bytes(info: PrefillPlanInfo, head_dim: int, host_only: bool = False) -> int:
    lib = _capi.load(host_only=host_only)
    return int(lib.pkv_prefill_workspace_bytes(C.byref(info), head_dim))


def decode_plan(context_lens: np.ndarray, partition_tokens: int = 0, block_size: int = 16,
                host_only: bool = False) -> Tuple[np.ndarray, PlanInfo]:
    """Host split-K plan (see pkv_decode_plan) for these context lengths."""
    lib = _capi.load(host_only=host_only)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    n = C.c_int32()
    check(lib, lib.pkv_decode_plan_ints(i32p(lens), len(lens), block_size, partition_tokens,
                                        C.byref(n)))
    plan = np.empty(max(n.value, 1), dtype=np.int32)
    info = PlanInfo()
    check(lib, lib.pkv_decode_plan(i32p(lens), len(lens), block_size, partition_tokens, i32p(plan),
                                   len(plan), C.byref(info)))
    return plan[:info.plan_ints], info


def decode_plan_shared(pool: "Pool", seqs, num_q_heads: int, partition_tokens: int = 0,
                       chunk_tokens: int = 0) -> Tuple[np.ndarray, PlanInfo]:
    """Split-K plan of live sequences of ``pool`` that reads blocks held in
    common once for all their holders (see pkv_decode_plan_shared)."""
    lib = pool.lib
    seqs_np = np.ascontiguousarray(seqs, dtype=np.int32)
    n = C.c_int32()
    check(lib, lib.pkv_decode_plan_shared_ints(pool.handle, i32p(seqs_np), len(seqs_np), partition_tokens,
                                               C.byref(n)))
    plan = np.empty(max(n.value, 1), dtype=np.int32)
    info = PlanInfo()
    check(lib, lib.pkv_decode_plan_shared(pool.handle, i32p(seqs_np), len(seqs_np), partition_tokens,
                                          num_q_heads, chunk_tokens, i32p(plan), len(plan), C.byref(info)))
    return plan[:info.plan_ints], info


def decode_workspace_bytes(info: PlanInfo, num_q_heads: int, head_dim: int,
                           host_only: bool = False) -> int:
    lib = _capi.load(host_only=host_only)
    return int(lib.pkv_decode_workspace_bytes(C.byref(info), num_q_heads, head_dim))


def decode_workspace_bound(max_seqs: int, max_context_len: int, num_q_heads: int, head_dim: int,
                           partition_tokens: int = 0, block_size: int = 16,
                           host_only: bool = False) -> int:
    """Workspace bytes enough for any batch within these limits."""
    lib = _capi.load(host_only=host_only)
    n = int(lib.pkv_decode_workspace_bound(max_seqs, max_context_len, block_size, partition_tokens,
                                           num_q_heads, head_dim))
    if n == 0:
        raise ValueError("bad decode geometry")
    return n


def fill_partition(context_lens, workgroups_per_item: int, resident: int, min_tokens: int = 512,
                   block_size: int = 16, host_only: bool = False) -> int:
    """Smallest multiple of block_size >= min_tokens whose split-K plan puts
    at most `resident` workgroups in flight (0 if none does)."""
    lib = _capi.load(host_only=host_only)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    return int(lib.pkv_decode_fill_partition(i32p(lens), len(lens), block_size, workgroups_per_item,
                                             int(resident), min_tokens))


def default_partition_tokens(host_only: bool = False) -> int:
    return int(_capi.load(host_only=host_only).pkv_default_partition_tokens())
