"""Shared test helpers for block allocators (the oracle's and the C++ one).

An adapter exposes: alloc(n) -> (id, slots), append(seq, n) -> slots,
append_batch(seqs, n) -> [slots], fork(seq) -> id, free(seq), take_cow() ->
[(src, dst)], table(seq), length(seq), live(), free_handout() -> [ids],
refcounts() -> [rc per block], stats() -> dict.  Errors raise an exception
with a ``kind`` attribute ("no_blocks", "bad_seq", "bad_arg", "table_full").
"""

from __future__ import annotations

import json
import os

import numpy as np


class OracleAdapter:
    def __init__(self, alloc):
        self.a = alloc

    def alloc(self, n):
        return self.a.alloc(n)

    def append(self, seq, n):
        return self.a.append(seq, n)

    def append_batch(self, seqs, n):
        return self.a.append_batch(seqs, n)

    def fork(self, seq):
        return self.a.fork(seq)

    def free(self, seq):
        self.a.free_seq(seq)

    def take_cow(self):
        return self.a.take_cow()

    def table(self, seq):
        return self.a.table(seq)

    def length(self, seq):
        return self.a.length(seq)

    def live(self):
        return self.a.live()

    def free_handout(self):
        return self.a.free_handout_order()

    def refcounts(self):
        return list(self.a.rc)

    def stats(self):
        return self.a.stats()


def load_trace(golden_dir, name="alloc_trace_bs4.json"):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def run_trace(adapter, trace):
    """Replay a golden trace step by step, asserting every expectation."""
    for i, step in enumerate(trace["steps"]):
        op, exp = step["op"], step["expect"]
        ctx = f"step {i} ({op})"
        result, err = None, None
        try:
            if op == "alloc":
                result = adapter.alloc(step["n"])
            elif op == "fork":
                result = adapter.fork(step["seq"])
            elif op == "append":
                result = adapter.append(step["seq"], step["n"])
            elif op == "append_batch":
                result = adapter.append_batch(step["seqs"], step["n"])
            elif op == "free":
                result = adapter.free(step["seq"])
            elif op == "take_cow":
                result = adapter.take_cow()
            else:
                raise AssertionError(f"unknown op {op}")
        except Exception as e:  # noqa: BLE001 -- error kinds are compared below
            err = getattr(e, "kind", None) or repr(e)
        if "error" in exp:
            assert err == exp["error"], f"{ctx}: expected error {exp['error']}, got {err}"
        else:
            assert err is None, f"{ctx}: unexpected error {err}"
        if "seq" in exp:
            sid = result[0] if op == "alloc" else result
            assert sid == exp["seq"], ctx
        if "slots" in exp:
            got = result[1] if op == "alloc" else result
            assert [list(x) if isinstance(x, (list, tuple)) else x for x in got] == exp["slots"], ctx
        if "pairs" in exp:
            assert [list(p) for p in result] == exp["pairs"], ctx
        if "free" in exp:
            assert adapter.free_handout() == exp["free"], ctx
        if "rc" in exp:
            rc = adapter.refcounts()
            for b, want in exp["rc"].items():
                assert rc[int(b)] == want, f"{ctx}: rc[{b}]"
        if "tables" in exp:
            want = {int(k): v for k, v in exp["tables"].items()}
            assert adapter.live() == sorted(want), ctx
            for sid, (table, length) in want.items():
                assert adapter.table(sid) == table, f"{ctx}: table of {sid}"
                assert adapter.length(sid) == length, f"{ctx}: length of {sid}"
        if "stats" in exp:
            st = adapter.stats()
            for k, v in exp["stats"].items():
                assert st[k] == v, f"{ctx}: stats[{k}] = {st[k]} != {v}"


def check_invariants(adapter, num_blocks, block_size):
    """Properties the pages state, checked on the full allocator state."""
    free = adapter.free_handout()
    rc = adapter.refcounts()
    live = adapter.live()
    # free list holds distinct blocks, exactly those with refcount 0
    assert len(set(free)) == len(free)
    assert set(free) == {b for b in range(num_blocks) if rc[b] == 0}
    # refcount = number of live tables holding the block
    holders = np.zeros(num_blocks, dtype=np.int64)
    waste = 0
    for sid in live:
        t = adapter.table(sid)
        L = adapter.length(sid)
        assert len(set(t)) == len(t)
        assert len(t) == -(-L // block_size)
        w = block_size * len(t) - L
        assert 0 <= w <= block_size - 1  # bounded internal fragmentation
        waste += w
        for b in t:
            holders[b] += 1
    assert list(holders) == rc
    st = adapter.stats()
    assert st["free_blocks"] == len(free)
    assert st["used_blocks"] == num_blocks - len(free)
    assert st["tail_waste_slots"] == waste
    assert st["shared_blocks"] == int(np.sum(np.asarray(rc) > 1))
