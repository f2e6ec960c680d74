"""The host chunked-prefill work list (pkv_prefill_plan), checked by enumeration (CPU).

Every (sequence, tile) appears; a tile's stages (32 keys each, up to the
keys its last query attends) are covered exactly once by its parts; a split
tile's parts are balanced and at most max_keys keys each; items are sorted
by the keys they attend, largest first (a launch of at most 512 workgroups:
the second half in increasing order); q_start are the prefix sums of the
chunk lengths; the split table points at disjoint, consecutive partials.
"""

import numpy as np
import pytest

from paged_kv_cache_257_amd import PkvError, prefill_plan, prefill_workspace_bytes
from workloads.prefill import PREFILL_CONFIGS, draw_prefill_shapes


def tile_for(Hq, Hkv):
    G = Hq // Hkv
    gw = 1
    while gw < 16 and G % (2 * gw) == 0:
        gw *= 2
    return 128 // gw, gw


def check(q_lens, ctx, Hq, Hkv, max_keys=0):
    plan, info = prefill_plan(q_lens, ctx, Hq, Hkv, max_keys, host_only=True)
    B = len(q_lens)
    tile, gw = tile_for(Hq, Hkv)
    assert info.tile_tokens == tile
    nw = info.n_work
    items = plan[:6 * nw].reshape(nw, 6)
    q_start = plan[6 * nw:6 * nw + B + 1]
    split_tab = plan[6 * nw + B + 1:].reshape(-1, 2)
    assert q_start.tolist() == [0] + np.cumsum(q_lens).tolist()
    assert len(split_tab) == info.n_split
    tiles = {}
    for seq, t, s0, s1, sp, part in items.tolist():
        tiles.setdefault((seq, t), []).append((s0, s1, sp, part))
    want = {(i, j) for i in range(B) for j in range(-(-int(q_lens[i]) // tile))}
    assert set(tiles) == want
    pos = 0
    for (seq, t), parts in sorted(tiles.items(), key=lambda kv: min(p[2] for p in kv[1])):
        C = int(ctx[seq]) - int(q_lens[seq])
        keys = C + min((t + 1) * tile, int(q_lens[seq]))
        stages = -(-keys // 32)
        parts = sorted(parts)
        assert parts[0][0] == 0 and parts[-1][1] == stages
        for a, b in zip(parts, parts[1:]):
            assert a[1] == b[0]
        if len(parts) == 1:
            assert parts[0][2] == -1 and (max_keys <= 0 or keys <= max_keys)
        else:
            assert max_keys > 0 and keys > max_keys
            sp = parts[0][2]
            assert all(p[2] == sp for p in parts) and [p[3] for p in parts] == list(range(len(parts)))
            assert split_tab[sp].tolist() == [pos, len(parts)]
            pos += len(parts)
            sizes = [p[1] - p[0] for p in parts]
            assert max(sizes) * 32 <= max(max_keys, 32) and max(sizes) - min(sizes) <= 1
    assert info.n_partials == pos
    cost = [min(s1 * 32, int(ctx[seq]) - int(q_lens[seq]) + min((t + 1) * tile, int(q_lens[seq])))
            if sp < 0 else (s1 - s0) * 32 for seq, t, s0, s1, sp, _ in items.tolist()]
    wgs = nw * Hkv * (Hq // Hkv // gw)
    if wgs <= 512:  # one round: the second half ascending, paired with the first on the CUs
        h = nw // 2
        assert cost[:h] == sorted(cost[:h], reverse=True) and cost[h:] == sorted(cost[h:])
        assert sorted(cost, reverse=True) == cost[:h] + cost[h:][::-1]
    else:
        assert cost == sorted(cost, reverse=True)
    assert info.total_q == int(np.sum(q_lens)) and info.max_context_len == int(max(ctx))
    assert info.plan_ints == len(plan)
    return info


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (32, 8), (12, 4), (48, 2), (6, 1)])
@pytest.mark.parametrize("max_keys", [0, 100, 1024])
def test_plan_enumerates_tiles_longest_first(Hq, Hkv, max_keys):
    rng = np.random.default_rng(Hq * 10 + Hkv)
    q_lens = rng.integers(1, 300, size=9)
    ctx = q_lens + rng.integers(0, 5000, size=9)
    info = check(q_lens, ctx, Hq, Hkv, max_keys)
    if max_keys == 100:
        assert info.n_split > 0


def test_plan_for_every_workload_step():
    for cfg in PREFILL_CONFIGS:
        sh = draw_prefill_shapes(cfg)
        for step in sh.steps:
            q_lens = np.array([n for _, _, n in step])
            ctx = np.array([t0 + n for _, t0, n in step])
            for mk in (0, 4096):
                check(q_lens, ctx, cfg.num_q_heads, cfg.num_kv_heads, mk)


def test_auto_split_fills_underfilled_launches():
    # 2048-token chunk of one prompt, 32 heads: 16 tiles x 32 = 512 workgroups, no split
    _, info = prefill_plan([2048], [30000], 32, 32, -1, host_only=True)
    assert info.n_split == 0
    # a 256-token slice: 2 tiles x 32 = 64 workgroups -> split to about 512
    plan, info = prefill_plan([256], [30000], 32, 32, -1, host_only=True)
    assert info.n_split == 2 and 512 <= info.n_work * 32 <= 640
    check([256], [30000], 32, 32, max_keys=30000 // 8)  # explicit limit of the same size
    # a short context never splits below 1024 keys per part
    _, info = prefill_plan([40], [1500], 4, 4, -1, host_only=True)
    assert info.n_work <= 2


def test_workspace_bytes():
    plan, info = prefill_plan([300], [9000], 32, 8, 1024, host_only=True)
    tile, gw = tile_for(32, 8)
    hgroups = 8 * (4 // gw)
    tickets = -(-info.n_split * hgroups * 4 // 256) * 256
    assert prefill_workspace_bytes(info, 128, host_only=True) == tickets + info.n_partials * hgroups * 128 * 640
    _, info0 = prefill_plan([300], [9000], 32, 8, 0, host_only=True)
    assert info0.n_split == 0 and prefill_workspace_bytes(info0, 128, host_only=True) == 0


def test_plan_errors():
    with pytest.raises(PkvError):
        prefill_plan([0], [5], 4, 4, host_only=True)
    with pytest.raises(PkvError):
        prefill_plan([6], [5], 4, 4, host_only=True)
    with pytest.raises(PkvError):
        prefill_plan([3], [5], 6, 4, host_only=True)
    plan, info = prefill_plan([], [], 4, 4, host_only=True)
    assert info.n_work == 0 and plan.tolist() == [0]
