"""Iteration-level continuous-batching scheduler (oracle; test infrastructure only).

"PagedAttention e continuous batching", 01 · Conceito: the batch is
revisited at every iteration boundary (finished sequences leave, waiting
ones enter, running ones advance one token); the scheduler weighs free
blocks, the tokens of a batch and the prefill/decode mix, slicing long
prefills; admission is decided in blocks, so a request that cannot fit is
turned away before it starts (the scheduler paragraph); preemptions, prefix hits, queue
delay, time to first token and inter-token latency are among the metrics
to keep (the metrics paragraph).  The rules are readings, in this order
per iteration t:

  1. requests arriving at t join the back of the waiting queue (id order);
  2. each running sequence past its prefill needs room for one more token,
     and the oldest running sequence still in prefill needs room for its
     next slice; while those needs exceed the free blocks, preempt the most
     recently admitted running sequence (for the slice, never that prefill
     itself or an older one; for the decodes, whichever is newest): free
     it, put it at the front of the queue; when readmitted it prefills
     again over prompt + generated - 1 tokens.  The oldest running request
     therefore always advances (slices of several prefills cannot hold all
     blocks while waiting on each other);
  3. those sequences each append one token and generate one;
  4. with budget = max_batch_tokens - decode tokens, running prefills take
     min(rest, chunk, budget) tokens in admission order, stopping at the
     first whose slice does not fit in the free blocks;
  5. while budget > 0, requests wait and fewer than max_running run: reject
     the head if its final length can never fit (more blocks than the pool
     or a table); else admit it if its first slice fits, else stop.  If a
     running sequence of the same prefix id has prefilled the prefix, fork
     those prefix tokens and prefill the rest;
  6. a completed first prefill generates the first token; requests with
     all their tokens finish; their sequences stay allocated until the start
     of the next iteration (0.), so that this iteration's items stay valid
     while the device runs them.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

from .allocator import OracleAllocator

PREFILL, DECODE = 0, 1
PENDING, WAITING, RUNNING, FINISHED, REJECTED = range(5)


@dataclass
class OracleRequest:
    arrival: int
    prompt_len: int
    output_len: int
    klass: int = 0
    prefix_id: int = -1
    prefix_len: int = 0
    # state
    state: int = PENDING
    seq: int = -1
    admitted_at: int = -1
    first_token_at: int = -1
    finished_at: int = -1
    generated: int = 0
    preemptions: int = 0
    prefix_hit_tokens: int = 0
    prefilled: int = 0
    target: int = 0


class OracleScheduler:
    def __init__(self, alloc: OracleAllocator, max_batch_tokens: int, chunk_tokens: int,
                 max_running: int, requests: List[OracleRequest]):
        self.a = alloc
        self.max_batch_tokens = max_batch_tokens
        self.chunk = chunk_tokens
        self.max_running = max_running
        self.reqs = requests
        for r in self.reqs:
            if r.prefix_id < 0:
                r.prefix_len = 0
        self.pending = sorted(range(len(requests)), key=lambda i: (requests[i].arrival, i))
        self.waiting: deque = deque()
        self.running: List[int] = []
        self.retired: List[int] = []
        self.holder: Dict[int, int] = {}
        self.t = 0
        self.stats = dict(preemptions=0, rejected=0, finished=0, prompt_tokens_admitted=0,
                          prefix_hit_tokens=0, prefill_tokens=0, decode_tokens=0)

    # ---- helpers -------------------------------------------------------------
    def _free_blocks(self) -> int:
        return len(self.a.free)

    def _need(self, seq: int, n: int) -> int:
        bs = self.a.block_size
        L = self.a.length(seq)
        table = self.a.table(seq)
        need = -(-(L + n) // bs) - len(table)
        if n > 0 and L % bs and self.a.rc[table[-1]] > 1:
            need += 1
        return need

    def _decoding(self, r: OracleRequest) -> bool:
        return r.prefilled == r.target and r.generated < r.output_len

    def _drop_holder(self, i: int) -> None:
        r = self.reqs[i]
        if r.prefix_id < 0 or self.holder.get(r.prefix_id) != i:
            return
        for j in self.running:
            q = self.reqs[j]
            if j != i and q.prefix_id == r.prefix_id and q.prefilled >= q.prefix_len:
                self.holder[r.prefix_id] = j
                return
        del self.holder[r.prefix_id]

    def _note(self, i: int) -> None:
        r = self.reqs[i]
        if r.prefix_id >= 0 and r.prefix_len > 0 and r.prefilled >= r.prefix_len \
                and r.prefix_id not in self.holder:
            self.holder[r.prefix_id] = i

    def _victim(self) -> int:
        """Rule 2: the running request preempted first, the most recently
        admitted one."""
        return self.running[-1]

    def _recompute_target(self, r: OracleRequest) -> int:
        """Rule 2: tokens a (re)admitted request prefills, its prompt plus every
        generated token but the newest, whose K/V the next decode appends."""
        return r.prompt_len + max(r.generated - 1, 0)

    def _prefill_done(self, r: OracleRequest) -> None:
        if r.generated == 0:
            r.generated = 1
            r.first_token_at = self.t

    # ---- one iteration -------------------------------------------------------
    def step(self):
        """Returns (items [(request, seq, kind, pos, n)], events dict)."""
        bs = self.a.block_size
        items: List[Tuple[int, int, int, int, int]] = []
        ev = dict(iteration=self.t, prefill_tokens=0, decode_tokens=0, admitted=0, preempted=0,
                  finished=0, rejected=0)
        for i in self.retired:
            self.a.free_seq(self.reqs[i].seq)
            self.reqs[i].seq = -1
        self.retired = []
        while self.pending and self.reqs[self.pending[0]].arrival <= self.t:
            i = self.pending.pop(0)
            self.reqs[i].state = WAITING
            self.waiting.append(i)

        while self.running:
            dec = [i for i in self.running if self._decoding(self.reqs[i])]
            dec_need = sum(self._need(self.reqs[i].seq, 1) for i in dec)
            pf = [i for i in self.running
                  if not self._decoding(self.reqs[i]) and self.reqs[i].prefilled < self.reqs[i].target]
            first = pf[0] if pf else None
            pf_need = 0
            if first is not None:
                r0 = self.reqs[first]
                n = min(r0.target - r0.prefilled, self.chunk, self.max_batch_tokens - len(dec))
                if n > 0:
                    pf_need = self._need(r0.seq, n)
            free = self._free_blocks()
            # the decodes' room may displace any newest sequence; the oldest
            # prefill's slice only sequences newer than it
            if dec_need <= free and (dec_need + pf_need <= free or self.running[-1] == first):
                break
            v = self._victim()
            r = self.reqs[v]
            self._drop_holder(v)
            self.a.free_seq(r.seq)
            self.running.remove(v)
            r.seq, r.state, r.prefilled = -1, WAITING, 0
            r.preemptions += 1
            self.waiting.appendleft(v)
            self.stats["preemptions"] += 1
            ev["preempted"] += 1

        for i in self.running:
            r = self.reqs[i]
            if not self._decoding(r):
                continue
            pos = r.prefilled
            self.a.append(r.seq, 1)
            r.prefilled += 1
            r.target += 1
            r.generated += 1
            items.append((i, r.seq, DECODE, pos, 1))
            ev["decode_tokens"] += 1
        budget = self.max_batch_tokens - ev["decode_tokens"]

        for i in self.running:
            if budget <= 0:
                break
            r = self.reqs[i]
            if r.prefilled >= r.target:
                continue
            n = min(r.target - r.prefilled, self.chunk, budget)
            if self._need(r.seq, n) > self._free_blocks():
                break
            pos = r.prefilled
            self.a.append(r.seq, n)
            r.prefilled += n
            budget -= n
            ev["prefill_tokens"] += n
            items.append((i, r.seq, PREFILL, pos, n))
            self._note(i)
            if r.prefilled == r.target:
                self._prefill_done(r)

        while budget > 0 and self.waiting and len(self.running) < self.max_running:
            i = self.waiting[0]
            r = self.reqs[i]
            final_blocks = -(-(r.prompt_len + r.output_len - 1) // bs)
            if final_blocks > self.a.num_blocks or final_blocks > self.a.max_blocks_per_seq:
                self.waiting.popleft()
                r.state = REJECTED
                self.stats["rejected"] += 1
                ev["rejected"] += 1
                continue
            target = self._recompute_target(r)
            h = self.holder.get(r.prefix_id) if r.prefix_id >= 0 and r.prefix_len > 0 else None
            start = r.prefix_len if h is not None else 0
            n = min(target - start, self.chunk, budget)
            need = -(-(start + n) // bs) - (-(-start // bs))
            if need > self._free_blocks():
                break
            if start:
                seq = self.a.fork_prefix(self.reqs[h].seq, start)
                self.a.append(seq, n)
            else:
                seq, _ = self.a.alloc(n)
            self.waiting.popleft()
            self.running.append(i)
            r.state, r.seq = RUNNING, seq
            if r.admitted_at < 0:
                r.admitted_at = self.t
            r.prefix_hit_tokens += start
            r.prefilled, r.target = start + n, target
            self.stats["prompt_tokens_admitted"] += target
            self.stats["prefix_hit_tokens"] += start
            budget -= n
            ev["prefill_tokens"] += n
            ev["admitted"] += 1
            items.append((i, seq, PREFILL, start, n))
            self._note(i)
            if r.prefilled == r.target:
                self._prefill_done(r)

        for i in list(self.running):
            r = self.reqs[i]
            if r.prefilled == r.target and r.generated >= r.output_len:
                self._drop_holder(i)
                self.retired.append(i)
                r.state, r.finished_at = FINISHED, self.t
                self.running.remove(i)
                self.stats["finished"] += 1
                ev["finished"] += 1

        self.stats["prefill_tokens"] += ev["prefill_tokens"]
        self.stats["decode_tokens"] += ev["decode_tokens"]
        self.t += 1
        return items, ev

    def done(self) -> bool:
        """Every request finished or rejected (a last step frees the last
        finished sequences)."""
        return not self.pending and not self.waiting and not self.running
