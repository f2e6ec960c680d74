"""The host split-K plan (pkv_decode_plan), checked by enumeration (CPU)."""

import numpy as np
import pytest

from paged_kv_cache_257_amd import (PkvError, decode_plan, decode_workspace_bound,
                                    decode_workspace_bytes, default_partition_tokens)
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
    # tight when every sequence has the maximum length
    lens = np.full(9, 5000)
    _, info = decode_plan(lens, 0, host_only=True)
    assert decode_workspace_bound(9, 5000, 8, 128, 0, host_only=True) == \
        decode_workspace_bytes(info, 8, 128, host_only=True)
    with pytest.raises(ValueError):
        decode_workspace_bound(4, 100, 8, 128, 24, host_only=True)
