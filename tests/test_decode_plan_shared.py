"""The shared-block decode plan (pkv_decode_plan_shared), on the CPU.

Sequences forked from one prompt point at the same read-only blocks
("PagedAttention e continuous batching", 01 · Conceito, paragraph 6); the
plan groups such blocks into nodes read once for all their holders.  Pinned
here by enumeration and by the oracle's split-K identity:
  * every block of every sequence is covered exactly once, by the chunks of
    the nodes it belongs to or by its own partitions; node members hold the
    node's blocks at the same table positions and never their last block;
    record indices are distinct, contiguous and capped;
  * attention assembled from the plan's pieces (one fp64 partial per node
    chunk and member, one per private partition, merged with the oracle's
    combine) equals the oracle's attention over the whole sequence;
  * below a quarter of shared context, or for pools the shared kernel does
    not take, the plan is pkv_decode_plan's with the load-policy hint.
"""

import numpy as np
import pytest

from oracle.attention import combine_partials, decode_attention, decode_partials
from paged_kv_cache_257_amd import Pool, _capi, decode_plan, decode_plan_shared

BS = 16


def forked_batch(rng, prefix_tokens=320, n_forks=40, tail_max=100, lineages=10, nb=900, kv_heads=2,
                 dtype="f16", head_dim=128, width=64):
    pool = Pool(nb, kv_heads, head_dim, dtype, width, BS, rng.permutation(nb).astype(np.int32), host_only=True)
    root, _ = pool.alloc(prefix_tokens)
    seqs = []
    for _ in range(n_forks):
        c = pool.fork(root)
        t = int(rng.integers(0, tail_max + 1))
        if t:
            pool.append(c, t)
        seqs.append(c)
    # lineages: forks of forks (they share the parent's tail blocks too)
    for _ in range(lineages):
        par = seqs[int(rng.integers(0, len(seqs)))]
        c = pool.fork(par)
        pool.append(c, int(rng.integers(1, 40)))
        seqs.append(c)
    for s in seqs:  # the decode token: the last block becomes the sequence's own
        pool.append(s, 1)
    pool.take_cow()
    return pool, seqs


def sections(plan, info, n):
    nw = info.n_work
    work = plan[:2 * nw].reshape(nw, 2)
    part_offset = plan[2 * nw:2 * nw + n]
    if info.n_nodes == 0:
        return work, part_offset, np.zeros(n, np.int64), np.zeros(n, np.int64), None, None
    sec = plan[info.off_shared:]
    priv, nsh, order = sec[:n], sec[n:2 * n], sec[2 * n:3 * n]
    nodes = sec[3 * n:3 * n + 9 * info.n_nodes].reshape(info.n_nodes, 9)
    return work, part_offset, priv, nsh, order, nodes


def check_plan(pool, seqs, plan, info, P, group, chunk_fixed=False):
    n = len(seqs)
    tabs = [pool.table(s) for s in seqs]
    nblk = [len(t) for t in tabs]
    work, part_offset, priv, nsh, order, nodes = sections(plan, info, n)
    cover = [np.zeros(b, np.int64) for b in nblk]
    recs = [[] for _ in range(n)]
    if info.n_nodes:
        assert sorted(order.tolist()) == list(range(n))
        items = [0, 0]
        for v, (rep, j0, j1, first, mem, kb, fi, cs, cb) in enumerate(nodes.tolist()):
            narrow = v >= info.n_wide_nodes
            assert narrow == (mem * group <= 16)  # wide nodes first
            assert cb >= (info.narrow_chunk_blocks if narrow else info.shared_chunk_blocks)
            if chunk_fixed:
                assert cb == (info.narrow_chunk_blocks if narrow else info.shared_chunk_blocks)
            else:  # long nodes in at most 8 (wide) or 4 (narrow) chunks
                assert -(-(j1 - j0) // cb) <= (4 if narrow else 8)
            assert fi == items[narrow] and j0 < j1 and mem >= 2
            assert cs == (1 if narrow else -(-mem * group // 128))
            members = order[first:first + mem].tolist()
            assert rep in members
            nch = -(-(j1 - j0) // cb)
            items[narrow] += nch * cs
            for s in members:
                assert j1 <= nblk[s] - 1  # never a member's last block
                assert tabs[s][j0:j1] == tabs[rep][j0:j1]
                cover[s][j0:j1] += 1
                recs[s] += [kb + c for c in range(nch)]
        assert items == [info.n_shared_items, info.n_narrow_items]
    for i in range(n):
        assert sorted(recs[i]) == list(range(int(nsh[i])))
        assert nsh[i] <= _capi.MAX_SHARED_RECORDS
    pb = P // BS
    parts = [0] * n
    for s, q in work.tolist():
        b0 = int(priv[s]) + q * pb
        b1 = min(b0 + pb, nblk[s])
        assert b0 < b1
        cover[s][b0:b1] += 1
        parts[s] += 1
    assert all((c == 1).all() for c in cover)
    pos = 0
    for i in range(n):
        if nsh[i] + parts[i] > 1:
            assert part_offset[i] == pos
            pos += nsh[i] + parts[i]
        else:
            assert part_offset[i] == -1
    assert pos == info.n_partials


@pytest.mark.parametrize("group", [1, 4, 16])
@pytest.mark.parametrize("chunk", [0, 16, 64])
def test_shared_plan_covers_every_block_once(group, chunk):
    rng = np.random.default_rng(100 + group + chunk)
    pool, seqs = forked_batch(rng)
    try:
        for P in (32, 256, 2048):
            plan, info = decode_plan_shared(pool, seqs, group * pool.desc.num_kv_heads, P, chunk)
            assert info.n_nodes > 0 and info.shared_group == group and info.shared_kv == 0
            if chunk:
                assert info.shared_chunk_blocks == chunk // BS
                assert info.narrow_chunk_blocks == max(chunk // BS, 64)
            check_plan(pool, seqs, plan, info, P, group, chunk_fixed=chunk > 0)
    finally:
        pool.close()


def test_records_per_sequence_are_capped():
    """A deep chain of forks with one-block chunks would give a sequence one
    record per block; nodes stop at the cap and the rest is read privately."""
    rng = np.random.default_rng(3)
    pool = Pool(600, 1, 128, "f16", 64, BS, rng.permutation(600).astype(np.int32), host_only=True)
    try:
        s = pool.alloc(BS * 3)[0]
        chain = [s]
        for _ in range(15):  # each fork shares all earlier blocks, then grows by two blocks
            c = pool.fork(chain[-1])
            pool.append(c, 2 * BS)
            chain.append(c)
        for x in chain:
            pool.append(x, 1)
        pool.take_cow()
        # 16 query heads per KV head: every node is wide and takes the
        # one-block chunks asked for
        plan, info = decode_plan_shared(pool, chain, 16, 256, BS)
        assert info.n_nodes > 0 and info.n_wide_nodes == info.n_nodes
        nsh = plan[info.off_shared + len(chain):info.off_shared + 2 * len(chain)]
        assert nsh.max() == _capi.MAX_SHARED_RECORDS
        check_plan(pool, chain, plan, info, 256, 16, chunk_fixed=True)
    finally:
        pool.close()


def test_little_sharing_or_unsupported_pool_falls_back():
    rng = np.random.default_rng(4)
    # two forks of a short prompt among long private sequences: under a quarter
    pool = Pool(600, 2, 128, "f16", 64, BS, rng.permutation(600).astype(np.int32), host_only=True)
    try:
        p = pool.alloc(40)[0]
        seqs = [pool.fork(p), pool.fork(p)] + [pool.alloc(500)[0] for _ in range(4)]
        for s in seqs:
            pool.append(s, 1)
        pool.take_cow()
        plan, info = decode_plan_shared(pool, seqs, 2, 256)
        want, winfo = decode_plan(np.array([pool.length(s) for s in seqs]), 256, host_only=True)
        assert info.n_nodes == 0 and info.shared_kv == 0 and np.array_equal(plan, want)
    finally:
        pool.close()
    # heavily shared, but fp32 (or head_dim 64): no nodes, the cached-load hint instead
    for dtype, d in (("f32", 128), ("f16", 64)):
        pool, seqs = forked_batch(np.random.default_rng(5), dtype=dtype, head_dim=d)
        try:
            plan, info = decode_plan_shared(pool, seqs, 2, 256)
            assert info.n_nodes == 0 and info.shared_kv == 1
            want, _ = decode_plan(np.array([pool.length(s) for s in seqs]), 256, host_only=True)
            assert np.array_equal(plan, want)
        finally:
            pool.close()


def test_attention_from_plan_pieces_equals_whole_sequence():
    """fp64: per node chunk and member one partial over the chunk's tokens,
    per private partition one partial, merged with the oracle's combine ==
    the oracle's attention over the whole gathered sequence."""
    rng = np.random.default_rng(6)
    H, d, group = 2, 128, 2
    pool, seqs = forked_batch(rng, prefix_tokens=200, n_forks=12, tail_max=60, lineages=5, nb=300,
                              kv_heads=H, head_dim=d)
    try:
        K = rng.standard_normal((300, BS, H, d))
        V = rng.standard_normal((300, BS, H, d))
        Hq = H * group
        scale = 1 / np.sqrt(d)
        P = 48
        plan, info = decode_plan_shared(pool, seqs, Hq, P, BS * 2)
        assert info.n_nodes > 0
        n = len(seqs)
        work, part_offset, priv, nsh, order, nodes = sections(plan, info, n)
        tabs = [pool.table(s) for s in seqs]
        lens = [pool.length(s) for s in seqs]
        pieces = [[] for _ in range(n)]  # (first token, last token + 1)
        for rep, j0, j1, first, mem, kb, fi, cs, cb in nodes.tolist():
            for s in order[first:first + mem].tolist():
                for c in range(-(-(j1 - j0) // cb)):
                    lo = (j0 + c * cb) * BS
                    pieces[s].append((lo, min(j1 * BS, lo + cb * BS)))
        for s, q in work.tolist():
            lo = (int(priv[s]) + q * (P // BS)) * BS
            pieces[s].append((lo, min(lens[s], lo + P)))
        for i in range(n):
            rows = np.concatenate([np.arange(b * BS, b * BS + BS) for b in range(len(tabs[i]))])[:lens[i]]
            Ki = K[np.asarray(tabs[i])].reshape(-1, H, d)[:lens[i]]
            Vi = V[np.asarray(tabs[i])].reshape(-1, H, d)[:lens[i]]
            assert len(rows) == lens[i]
            q = rng.standard_normal((Hq, d))
            want = decode_attention(q, Ki, Vi, scale)
            ms, ls, os_ = [], [], []
            for lo, hi in sorted(pieces[i]):
                m_, l_, o_ = decode_partials(q, Ki[lo:hi], Vi[lo:hi], scale, hi - lo)
                ms.append(m_[0]), ls.append(l_[0]), os_.append(o_[0])
            got = combine_partials(np.array(ms), np.array(ls), np.array(os_))
            assert np.max(np.abs(got - want)) < 1e-12
    finally:
        pool.close()
