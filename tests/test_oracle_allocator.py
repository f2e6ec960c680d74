"""Pins for oracle/allocator.py and oracle/kvcache.py (CPU).

* a hand-worked trace (tests/golden/alloc_trace_bs4.json) pins the free-list
  order, copy-on-write, failures and statistics;
* the tiny workload's block counts and tail waste are the pages' arithmetic;
* seeded random operation sequences check, after every operation, the
  properties the pages state: no external fragmentation (an allocation
  succeeds exactly when enough blocks are free), at most block-1 wasted rows
  per sequence, freed blocks back on the free list, shared blocks carrying
  refcount > 1 until a divergent write copies them, nothing moving when a
  sequence grows, and the paged view equal to a dense never-paged shadow.
"""

import numpy as np
import pytest

from oracle.allocator import AllocError, OracleAllocator
from oracle.kvcache import DenseShadow, MirrorPool
from workloads import config_by_name
from workloads.configs import draw_decode_shapes
from tests.alloc_harness import OracleAdapter, check_invariants, load_trace, run_trace


def test_hand_worked_trace(golden_dir):
    trace = load_trace(golden_dir)
    p = trace["pool"]
    a = OracleAllocator(p["num_blocks"], p["block_size"], p["max_blocks_per_seq"], p["free_order"])
    run_trace(OracleAdapter(a), trace)


def test_tiny_workload_block_counts_and_waste():
    cfg = config_by_name("tiny_f32")
    sh = draw_decode_shapes(cfg)
    a = OracleAllocator(sh.num_blocks, 16, 8, sh.free_order)
    ids = [a.alloc(int(L))[0] for L in sh.lens]
    assert [len(a.table(i)) for i in ids] == [1, 2, 3, 4]
    assert a.stats()["used_blocks"] == 10 and sh.num_blocks == 32
    assert [16 * len(a.table(i)) - a.length(i) for i in ids] == [11, 15, 15, 4]
    # blocks come off the seeded permutation in order
    flat = [b for i in ids for b in a.table(i)]
    assert flat == list(sh.free_order[:10])


def test_alloc_succeeds_iff_enough_free_blocks():
    a = OracleAllocator(10, 16)
    a.alloc(16 * 7)
    free_before = a.free_handout_order()
    with pytest.raises(AllocError) as e:
        a.alloc(16 * 3 + 1)  # needs 4, 3 free
    assert e.value.kind == "no_blocks"
    assert a.free_handout_order() == free_before and a.stats()["alloc_failures"] == 1
    sid, _ = a.alloc(16 * 3)  # needs exactly 3
    assert a.stats()["free_blocks"] == 0
    assert sid == 1  # the failed call consumed no id


def test_table_full_is_refused_without_change():
    a = OracleAllocator(16, 16, max_blocks_per_seq=2)
    sid, _ = a.alloc(32)
    with pytest.raises(AllocError) as e:
        a.append(sid, 1)
    assert e.value.kind == "table_full"
    assert a.length(sid) == 32 and a.stats()["free_blocks"] == 14
    with pytest.raises(AllocError):
        a.alloc(33)
    assert a.stats()["free_blocks"] == 14


def test_shared_prefix_refcounts_until_divergence():
    a = OracleAllocator(64, 16)
    root, _ = a.alloc(40)  # 2 full blocks + 8 rows
    kids = [a.fork(root) for _ in range(3)]
    t = a.table(root)
    assert all(a.rc[b] == 4 for b in t)
    a.append(kids[0], 1)  # diverges inside the shared partial block
    pairs = a.take_cow()
    assert len(pairs) == 1 and pairs[0][0] == t[-1]
    assert a.table(kids[0])[:2] == t[:2] and a.table(kids[0])[2] == pairs[0][1]
    assert a.rc[t[0]] == 4 and a.rc[t[2]] == 3
    # a full shared block is never copied: the next token opens a new block
    b, _ = a.alloc(32)
    c = a.fork(b)
    a.append(c, 1)
    assert a.take_cow() == [] and a.table(c)[:2] == a.table(b)


def _fuzz_ops(seed, n_ops=400, num_blocks=48, bs=16, max_blocks=12):
    rng = np.random.default_rng(seed)
    a = OracleAllocator(num_blocks, bs, max_blocks, rng.permutation(num_blocks))
    ad = OracleAdapter(a)
    H, d = 2, 4
    mirror = MirrorPool(num_blocks, H, d, np.float32, bs)
    shadow = DenseShadow(H, d, np.float32)
    counter = [0]

    def rows(n):
        base = counter[0]
        counter[0] += n
        return (np.arange(base, base + n * H * d, dtype=np.float32).reshape(n, H, d),
                -np.arange(base, base + n * H * d, dtype=np.float32).reshape(n, H, d))

    def write(seq_slots):
        # copy-on-write copies happen before the new rows land
        mirror.copy_blocks(a.take_cow())
        for sid, slots in seq_slots:
            k, v = rows(len(slots))
            mirror.write_kv(k, v, slots)
            shadow.append(sid, k, v)

    for _ in range(n_ops):
        live = a.live()
        op = rng.choice(["alloc", "append", "batch", "fork", "free"], p=[.2, .3, .2, .15, .15])
        before = {s: a.table(s) for s in live}
        free_n = len(a.free)
        try:
            if op == "alloc":
                n = int(rng.integers(0, 80))
                need = -(-n // bs)
                sid, slots = a.alloc(n)
                assert need <= free_n
                shadow.new(sid)
                write([(sid, slots)])
            elif op == "append" and live:
                sid = int(rng.choice(live))
                n = int(rng.integers(1, 20))
                slots = a.append(sid, n)
                # nothing moves: old entries stay, except a copied last block
                old = before[sid]
                keep = len(old) - (1 if a.length(sid) - n < 16 * len(old) else 0)
                assert a.table(sid)[:keep] == old[:keep]
                write([(sid, slots)])
            elif op == "batch" and live:
                k = int(rng.integers(1, len(live) + 1))
                seqs = sorted(int(s) for s in rng.choice(live, k, replace=False))
                res = a.append_batch(seqs, 1)
                write(list(zip(seqs, res)))
            elif op == "fork" and live:
                p = int(rng.choice(live))
                c = a.fork(p)
                shadow.fork(p, c)
            elif op == "free" and live:
                sid = int(rng.choice(live))
                a.free_seq(sid)
                shadow.free(sid)
        except AllocError as e:
            assert e.kind in ("no_blocks", "table_full")
            assert {s: a.table(s) for s in a.live()} == before
            assert len(a.free) == free_n
        check_invariants(ad, num_blocks, bs)
        for sid in a.live():
            k, v = mirror.gather(a.table(sid), a.length(sid))
            ks, vs = shadow.get(sid)
            assert np.array_equal(k, ks) and np.array_equal(v, vs)
    return a


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_random_ops_keep_page_properties_and_dense_equality(seed):
    a = _fuzz_ops(seed)
    st = a.stats()
    assert st["forks"] > 0 and st["cow_copies"] > 0


def test_freeing_everything_returns_every_block():
    a = OracleAllocator(20, 16, free_order=list(range(19, -1, -1)))
    ids = [a.alloc(30)[0] for _ in range(5)]
    ids.append(a.fork(ids[0]))
    for s in ids:
        a.free_seq(s)
    assert sorted(a.free_handout_order()) == list(range(20))
    assert all(r == 0 for r in a.rc)
