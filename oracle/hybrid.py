"""Hybrid two-pool manager (oracle; test infrastructure only).

"PagedAttention e continuous batching", 01 · Conceito, paragraph 5: a
hybrid model pages the growing K/V of its attention layers, while its other
layers keep a recurrent state of fixed size per sequence, so the server
manages two pools with different lifecycles.  The model here: a state pool
of ``num_slots`` slots beside the paged K/V allocator.  Readings (the page
names the two pools, not their rules):
  * a sequence admitted through the manager holds its blocks and one slot;
  * a fork shares the parent's blocks (reference counts) but needs a slot
    of its own, filled with a copy of the parent's state, since that state
    changes every step; the copy (parent slot, child slot) is queued;
  * free returns the blocks and the slot;
  * admission and fork are all-or-nothing across both pools and refuse
    early ([lesson] paragraph 7): the slot is checked first, then blocks;
  * the slot free list is a stack seeded like the block free list.

Budget split ([lesson] paragraph 4's arithmetic): a session of T tokens
costs ceil(T / block) blocks plus one slot; sessions = floor(budget /
cost), the state pool gets that many slots and the K/V pool every whole
block left.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

from .allocator import NO_BLOCKS, TABLE_FULL, AllocError, OracleAllocator

NO_SLOTS = "no_slots"


class OracleHybrid:
    def __init__(self, kv: OracleAllocator, num_slots: int, slot_order: Optional[Sequence[int]] = None):
        order = list(range(num_slots)) if slot_order is None else [int(s) for s in slot_order]
        if sorted(order) != list(range(num_slots)):
            raise ValueError("slot_order must be a permutation of the slot ids")
        self.kv = kv
        self.num_slots = num_slots
        self.free_slots: List[int] = list(reversed(order))  # top = end = order[0]
        self.slot_of: Dict[int, int] = {}
        self.copies: List[Tuple[int, int]] = []
        self.refusals = 0
        self.state_copies = 0

    def admit(self, n_tokens: int):
        if not self.free_slots:
            self.refusals += 1
            raise AllocError(NO_SLOTS, "no free state slot")
        try:
            seq, slots = self.kv.alloc(n_tokens)
        except AllocError as e:
            if e.kind in (NO_BLOCKS, TABLE_FULL):
                self.refusals += 1
            raise
        slot = self.free_slots.pop()
        self.slot_of[seq] = slot
        return seq, slot, slots

    def fork(self, parent: int):
        if parent not in self.slot_of:
            raise AllocError("bad_seq", f"sequence {parent} is not held by this manager")
        if not self.free_slots:
            self.refusals += 1
            raise AllocError(NO_SLOTS, "no free state slot")
        child = self.kv.fork(parent)
        slot = self.free_slots.pop()
        self.slot_of[child] = slot
        self.copies.append((self.slot_of[parent], slot))
        self.state_copies += 1
        return child, slot

    def free(self, seq: int) -> None:
        if seq not in self.slot_of:
            raise AllocError("bad_seq", f"sequence {seq} is not held by this manager")
        self.kv.free_seq(seq)
        self.free_slots.append(self.slot_of.pop(seq))

    def take_copies(self) -> List[Tuple[int, int]]:
        out, self.copies = self.copies, []
        return out

    def stats(self) -> dict:
        return {"free_slots": len(self.free_slots), "used_slots": len(self.slot_of),
                "refusals": self.refusals, "state_copies": self.state_copies}


def plan_budget(budget_bytes: int, block_bytes: int, block_size: int, slot_bytes: int,
                session_tokens: int) -> Tuple[int, int, int]:
    """(sessions, K/V blocks, state slots) for a joint budget."""
    blocks_per_session = -(-session_tokens // block_size)
    cost = blocks_per_session * block_bytes + slot_bytes
    sessions = budget_bytes // cost
    blocks = (budget_bytes - sessions * slot_bytes) // block_bytes
    return sessions, blocks, sessions
