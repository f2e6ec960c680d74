"""Pure-Python paged block allocator (oracle; test infrastructure only).

Follows [preview] "La idea de PagedAttention":
  step 1  the KV cache is cut into fixed blocks of ``block_size`` tokens;
  step 2  each sequence keeps a block table: entry i is the physical block
          holding its logical block i;
  step 3  appending a token writes into the last block if it has room,
          otherwise a free block is taken and the table grows;
  step 4  freeing a sequence returns its blocks to a free list;
and [lesson] paragraph 6: sequences may point at the same read-only blocks
(forks, shared prefixes); when one of them diverges, copy-on-write gives the
writer a new block for the altered positions, and reference counts decide
when a shared block goes back to the pool.  [lesson] paragraph 7: admission
is decided in blocks, and a request that cannot fit is turned away at once
with an explicit error.

Readings (the pages leave these open):
  * free list = LIFO stack; its initial content is ``free_order`` and the
    first block handed out is ``free_order[0]``; ``free`` releases a table
    front to back, so a freed sequence's last block is reused first;
  * copy-on-write triggers when a token goes into a partly filled last block
    whose refcount is above 1: the writer takes a fresh block, a (src, dst)
    whole-block copy is queued, the source loses one reference; a full shared
    block is never copied (the next token opens a new block anyway);
  * every mutating call is all-or-nothing: on failure nothing changes, no id
    is consumed, and ``alloc_failures`` counts block shortages;
  * sequence ids count up from 0 and are never reused;
  * a batch append processes the listed sequences in the order given.
"""

from __future__ import annotations

import copy
from typing import Dict, List, Optional, Sequence, Tuple

NO_BLOCKS = "no_blocks"
BAD_SEQ = "bad_seq"
BAD_ARG = "bad_arg"
TABLE_FULL = "table_full"


class AllocError(Exception):
    def __init__(self, kind: str, msg: str):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind


class _Seq:
    __slots__ = ("table", "length")

    def __init__(self, table: List[int], length: int):
        self.table = table
        self.length = length


class OracleAllocator:
    def __init__(self, num_blocks: int, block_size: int = 16,
                 max_blocks_per_seq: Optional[int] = None,
                 free_order: Optional[Sequence[int]] = None):
        if num_blocks < 0 or block_size < 1:
            raise AllocError(BAD_ARG, "bad pool geometry")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise AllocError(BAD_ARG, "free_order must be a permutation of the block ids")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.max_blocks_per_seq = max_blocks_per_seq if max_blocks_per_seq else num_blocks
        self._initial_order = order
        self.reset()

    # ---- state -----------------------------------------------------------
    def reset(self) -> None:
        """Drop every sequence; the free list returns to its initial order."""
        self.free: List[int] = self._initial_order[::-1]  # top of stack = end
        self.rc: List[int] = [0] * self.num_blocks
        self.seqs: Dict[int, _Seq] = {}
        self.next_id = 0
        self.cow_pending: List[Tuple[int, int]] = []
        self.alloc_failures = 0
        self.cow_copies = 0
        self.forks = 0

    def _pop(self) -> int:
        b = self.free.pop()
        assert self.rc[b] == 0
        self.rc[b] = 1
        return b

    def _release(self, b: int) -> None:
        assert self.rc[b] > 0
        self.rc[b] -= 1
        if self.rc[b] == 0:
            self.free.append(b)

    def _get(self, seq: int) -> _Seq:
        s = self.seqs.get(int(seq))
        if s is None:
            raise AllocError(BAD_SEQ, f"unknown sequence {seq}")
        return s

    # ---- one token (preview step 3, lesson paragraph 6) ----------------------
    def _append_token(self, s: _Seq) -> int:
        bs = self.block_size
        L = s.length
        if L % bs == 0:
            if len(s.table) >= self.max_blocks_per_seq:
                raise AllocError(TABLE_FULL, "block table is full")
            if not self.free:
                raise AllocError(NO_BLOCKS, "no free block")
            s.table.append(self._pop())
        else:
            last = s.table[-1]
            if self.rc[last] > 1:
                if not self.free:
                    raise AllocError(NO_BLOCKS, "no free block for copy-on-write")
                fresh = self._pop()
                self.cow_pending.append((last, fresh))
                self.cow_copies += 1
                self.rc[last] -= 1  # still > 0: someone else holds it
                s.table[-1] = fresh
        slot = s.table[L // bs] * bs + L % bs
        s.length = L + 1
        return slot

    def _transaction(self, fn):
        """Run fn on the live state; on AllocError restore everything."""
        saved = (list(self.free), list(self.rc), copy.deepcopy(self.seqs), self.next_id,
                 list(self.cow_pending), self.cow_copies, self.forks)
        try:
            return fn()
        except AllocError as e:
            (self.free, self.rc, self.seqs, self.next_id, self.cow_pending,
             self.cow_copies, self.forks) = saved
            if e.kind == NO_BLOCKS:
                self.alloc_failures += 1
            raise

    # ---- public API -------------------------------------------------------
    def alloc(self, n_tokens: int) -> Tuple[int, List[int]]:
        """New sequence holding n tokens; returns (id, slots of its tokens)."""
        if n_tokens < 0:
            raise AllocError(BAD_ARG, "negative token count")

        def run():
            sid = self.next_id
            s = _Seq([], 0)
            slots = [self._append_token(s) for _ in range(n_tokens)]
            self.seqs[sid] = s
            self.next_id += 1
            return sid, slots

        return self._transaction(run)

    def append(self, seq: int, n_tokens: int = 1) -> List[int]:
        if n_tokens < 0:
            raise AllocError(BAD_ARG, "negative token count")

        def run():
            s = self._get(seq)
            return [self._append_token(s) for _ in range(n_tokens)]

        return self._transaction(run)

    def append_batch(self, seqs: Sequence[int], n_tokens: int = 1) -> List[List[int]]:
        """Append n tokens to each listed sequence, in list order, atomically."""
        if len(set(int(s) for s in seqs)) != len(seqs):
            raise AllocError(BAD_ARG, "duplicate sequence in batch")

        def run():
            out = []
            for sid in seqs:
                s = self._get(sid)
                out.append([self._append_token(s) for _ in range(n_tokens)])
            return out

        return self._transaction(run)

    def fork(self, parent: int) -> int:
        """New sequence sharing every block of ``parent`` (refcounts + 1)."""
        p = self._get(parent)
        for b in p.table:
            self.rc[b] += 1
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = _Seq(list(p.table), p.length)
        self.forks += 1
        return sid

    def fork_prefix(self, parent: int, n_tokens: int) -> int:
        """New sequence sharing the first n_tokens tokens of ``parent``: its
        table is the parent's first ceil(n / block) blocks (refcounts + 1)."""
        p = self._get(parent)
        if n_tokens < 0 or n_tokens > p.length:
            raise AllocError(BAD_ARG, "prefix longer than the parent")
        table = p.table[:-(-n_tokens // self.block_size)] if n_tokens else []
        for b in table:
            self.rc[b] += 1
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = _Seq(list(table), n_tokens)
        self.forks += 1
        return sid

    def free_seq(self, seq: int) -> None:
        s = self._get(seq)
        del self.seqs[int(seq)]
        for b in s.table:
            self._release(b)

    def take_cow(self) -> List[Tuple[int, int]]:
        pairs, self.cow_pending = self.cow_pending, []
        return pairs

    # ---- views ------------------------------------------------------------
    def table(self, seq: int) -> List[int]:
        return list(self._get(seq).table)

    def length(self, seq: int) -> int:
        return self._get(seq).length

    def live(self) -> List[int]:
        return sorted(self.seqs)

    def free_handout_order(self) -> List[int]:
        """Free blocks in the order they would be handed out next."""
        return self.free[::-1]

    def build_batch(self, seqs: Sequence[int], width: int):
        """Block tables padded with -1 to ``width`` and context lengths."""
        tables, lens = [], []
        for sid in seqs:
            s = self._get(sid)
            if len(s.table) > width:
                raise AllocError(TABLE_FULL, "table wider than the batch stride")
            tables.append(s.table + [-1] * (width - len(s.table)))
            lens.append(s.length)
        return tables, lens

    def stats(self) -> dict:
        bs = self.block_size
        return dict(
            free_blocks=len(self.free),
            used_blocks=self.num_blocks - len(self.free),
            alloc_failures=self.alloc_failures,
            tail_waste_slots=sum(bs * len(s.table) - s.length for s in self.seqs.values()),
            shared_blocks=sum(1 for r in self.rc if r > 1),
            cow_copies=self.cow_copies,
            forks=self.forks,
            live_seqs=len(self.seqs),
        )
