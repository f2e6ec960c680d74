"""The host split-K plan (pkv_decode_plan), checked by enumeration (CPU)."""

import numpy as np
import pytest

from paged_kv_cache_257_amd import (PkvError, decode_plan, decode_workspace_bound,
                                    decode_workspace_bytes, default_partition_tokens, fill_partition)
from workloads import CONFIGS
from workloads.configs import draw_decode_shapes


def check_plan(lens, P):
    plan, info = decode_plan(lens, P, host_only=True)
    B = len(lens)
    nw = info.n_work
    work = plan[:2 * nw].reshape(nw, 2)
    offs = plan[2 * nw:2 * nw + B]
    red = plan[2 * nw + B:2 * nw + B + info.n_reduce]
    parts = [-(-int(L) // P) for L in lens]
    # every (seq, partition) exactly once
    want = sorted((i, p) for i in range(B) for p in range(parts[i]))
    assert sorted(map(tuple, work.tolist())) == want
    # longest first
    sizes = [min(P, int(lens[s]) - p * P) for s, p in work.tolist()]
    nblk = [-(-x // 16) for x in sizes]
    assert nblk == sorted(nblk, reverse=True)
    # partial offsets: contiguous ranges for multi-partition sequences only
    assert list(red) == [i for i in range(B) if parts[i] > 1]
    pos = 0
    for i in range(B):
        if parts[i] > 1:
            assert offs[i] == pos
            pos += parts[i]
        else:
            assert offs[i] == -1
    assert info.n_partials == pos and info.plan_ints == 2 * nw + B + info.n_reduce
    assert info.max_context_len == max(lens)
    return info


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
@pytest.mark.parametrize("P", [16, 256, 512])
def test_plan_covers_every_partition_once(cfg, P):
    sh = draw_decode_shapes(cfg)
    check_plan(sh.lens, P)


def test_plan_edge_cases():
    info = check_plan(np.array([1, 16, 17, 512, 513]), 256)
    assert info.n_reduce == 2
    tickets = -(-5 * 8 * 4 // 256) * 256  # one int32 per (sequence, query head), 256-byte aligned
    record = 640  # 128 + 2 floats, padded to whole 128-byte lines
    assert decode_workspace_bytes(info, 8, 128, host_only=True) == tickets + info.n_partials * 8 * record
    _, info0 = decode_plan(np.zeros(0, dtype=np.int32), 256, host_only=True)
    assert info0.n_work == 0
    with pytest.raises(PkvError):
        decode_plan(np.array([0]), 256, host_only=True)
    with pytest.raises(PkvError):
        decode_plan(np.array([5]), 24, host_only=True)


def test_default_partition_and_workspace_bound():
    P0 = default_partition_tokens(host_only=True)
    assert P0 > 0 and P0 % 16 == 0
    rng = np.random.default_rng(7)
    for trial in range(200):
        B = int(rng.integers(1, 40))
        Lmax = int(rng.integers(1, 20000))
        P = int(rng.choice([0, 16, 256, 2048]))
        lens = rng.integers(1, Lmax + 1, size=B)
        _, info = decode_plan(lens, P, host_only=True)
        assert info.partition_tokens == (P or P0)
        need = decode_workspace_bytes(info, 12, 64, host_only=True)
        for nb in (B, B + 3):
            assert decode_workspace_bound(nb, Lmax, 12, 64, P, host_only=True) >= need
    # when every sequence has the maximum length the bound is that plan's
    # workspace plus the shared records a shared-block plan may add (at
    # most PKV_MAX_SHARED_RECORDS per sequence, one per query head each)
    from paged_kv_cache_257_amd import _capi
    lens = np.full(9, 5000)
    _, info = decode_plan(lens, 0, host_only=True)
    record = 640  # o[128], m, l as fp32, padded to whole 128-byte lines
    assert decode_workspace_bound(9, 5000, 8, 128, 0, host_only=True) == \
        decode_workspace_bytes(info, 8, 128, host_only=True) + 9 * _capi.MAX_SHARED_RECORDS * 8 * record
    with pytest.raises(ValueError):
        decode_workspace_bound(4, 100, 8, 128, 24, host_only=True)


def _fill_brute(lens, wpi, resident, min_tokens, bs=16):
    """The rule restated by enumeration: the first multiple of bs >= min_tokens
    (up to the one holding the longest sequence whole) whose plan has at most
    `resident` workgroups, else 0."""
    lo = -(-min_tokens // bs)
    hi = max(lo, -(-max(lens) // bs)) if len(lens) else lo
    for m in range(lo, hi + 1):
        if wpi * sum(-(-int(L) // (m * bs)) for L in lens) <= resident:
            return m * bs
    return 0


def test_fill_partition_matches_enumeration():
    rng = np.random.default_rng(5)
    for _ in range(300):
        B = int(rng.integers(1, 40))
        lens = rng.integers(1, 40000, size=B).astype(np.int32)
        wpi = int(rng.choice([1, 2, 8, 32]))
        resident = int(rng.integers(1, 4000))
        mn = int(rng.choice([16, 256, 512, 1000]))
        assert fill_partition(lens, wpi, resident, mn, host_only=True) == _fill_brute(lens, wpi, resident, mn)


def test_fill_partition_cases():
    # 10 x 32,786 tokens, 8 workgroups per item, 768 resident (3 per CU on
    # 256 CUs): 9 partitions per sequence fit (720), 10 do not (800)
    lens = np.full(10, 32786, np.int32)
    P = fill_partition(lens, 8, 768, 512, host_only=True)
    assert P == 3648 and 8 * 10 * -(-32786 // P) <= 768 and 8 * 10 * -(-32786 // (P - 16)) > 768
    # 64 sequences x 32 heads cannot fit 768 at one partition each: 0
    assert fill_partition(np.full(64, 500, np.int32), 32, 768, 512, host_only=True) == 0
    # plenty of room: the minimum size
    assert fill_partition(np.array([5000], np.int32), 1, 10 ** 6, 512, host_only=True) == 512
    # a result is never below min_tokens, always a multiple of 16
    assert fill_partition(np.array([17], np.int32), 1, 1, 100, host_only=True) == 112
    # bad arguments -> 0
    assert fill_partition(np.array([0], np.int32), 1, 10, 512, host_only=True) == 0
    assert fill_partition(np.array([10], np.int32), 0, 10, 512, host_only=True) == 0


def test_fill_mode_sizes_buffers_for_its_minimum():
    from paged_kv_cache_257_amd import _capi
    lib = _capi.load(host_only=True)
    assert lib.pkv_prepare_decode_bytes(64, 1, 128, 16, -1) == lib.pkv_prepare_decode_bytes(64, 1, 128, 16, 512)
    assert decode_workspace_bound(10, 33000, 32, 128, partition_tokens=-1, host_only=True) == \
        decode_workspace_bound(10, 33000, 32, 128, partition_tokens=512, host_only=True)
