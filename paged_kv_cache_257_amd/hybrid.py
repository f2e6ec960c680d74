"""Python binding of the hybrid two-pool manager (pkv_hybrid_*): a paged
K/V pool plus fixed-size per-sequence state slots.  Marshalling only."""

from __future__ import annotations

import ctypes as C
from typing import Optional, Tuple

import numpy as np

from . import _capi
from ._capi import HybridStats, check, i32p, i64p
from .pool import Pool, _dptr, _stream_ptr


class Hybrid:
    def __init__(self, pool: Pool, num_slots: int, slot_bytes: int, state=None, slot_order=None):
        """``state``: optional device tensor of num_slots * slot_bytes bytes."""
        self.pool = pool
        self.lib = pool.lib
        self.num_slots, self.slot_bytes = int(num_slots), int(slot_bytes)
        self.state = state
        order = None if slot_order is None else np.ascontiguousarray(slot_order, dtype=np.int32)
        h = C.c_void_p()
        check(self.lib, self.lib.pkv_hybrid_create(pool.handle, self.num_slots, self.slot_bytes,
                                                   _dptr(state), None if order is None else i32p(order),
                                                   C.byref(h)))
        self.handle = h

    def close(self) -> None:
        if getattr(self, "handle", None):
            self.lib.pkv_hybrid_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 -- interpreter shutdown
            pass

    def admit(self, n_tokens: int) -> Tuple[int, int, np.ndarray]:
        seq, slot = C.c_int32(), C.c_int32()
        slots = np.empty(max(n_tokens, 1), dtype=np.int64)
        check(self.lib, self.lib.pkv_hybrid_admit(self.handle, n_tokens, C.byref(seq), C.byref(slot),
                                                  i64p(slots)))
        return seq.value, slot.value, slots[:n_tokens]

    def fork(self, parent: int) -> Tuple[int, int]:
        child, slot = C.c_int32(), C.c_int32()
        check(self.lib, self.lib.pkv_hybrid_fork(self.handle, parent, C.byref(child), C.byref(slot)))
        return child.value, slot.value

    def free(self, seq: int) -> None:
        check(self.lib, self.lib.pkv_hybrid_free(self.handle, seq))

    def slot(self, seq: int) -> int:
        s = C.c_int32()
        check(self.lib, self.lib.pkv_hybrid_slot(self.handle, seq, C.byref(s)))
        return s.value

    def take_copies(self) -> np.ndarray:
        n = C.c_int32()
        check(self.lib, self.lib.pkv_hybrid_take_copies(self.handle, None, 0, C.byref(n)))
        buf = np.empty((max(n.value, 1), 2), dtype=np.int32)
        check(self.lib, self.lib.pkv_hybrid_take_copies(self.handle, i32p(buf), n.value, C.byref(n)))
        return buf[:n.value]

    def stats(self) -> dict:
        s = HybridStats()
        check(self.lib, self.lib.pkv_hybrid_stats(self.handle, C.byref(s)))
        return s.as_dict()

    def copy_states(self, pairs, stream=None) -> None:
        """pairs: device int32 [n][2] (src slot, dst slot)."""
        check(self.lib, self.lib.pkv_hybrid_copy_states(self.handle, _dptr(pairs), int(pairs.shape[0]),
                                                        _stream_ptr(stream)))


def hybrid_plan(budget_bytes: int, block_bytes: int, block_size: int, slot_bytes: int,
                session_tokens: int, host_only: bool = False) -> Tuple[int, int, int]:
    """(sessions, K/V blocks, state slots) for a joint memory budget."""
    lib = _capi.load(host_only=host_only)
    a, b, c = C.c_int32(), C.c_int32(), C.c_int32()
    check(lib, lib.pkv_hybrid_plan(budget_bytes, block_bytes, block_size, slot_bytes, session_tokens,
                                   C.byref(a), C.byref(b), C.byref(c)))
    return a.value, b.value, c.value
