"""Seeded draws for the prefix-shared continuous-batching workload.

The workload: one root sequence holds a block-aligned shared prompt prefix;
``num_seqs`` sequences are forked from it and each appends its own tail of
``U[0, tail_max]`` tokens.  Each iteration then appends one token to every
live decoding sequence, decodes, retires ``churn`` seeded live sequences and
admits ``churn`` new ones as forks of seeded surviving sequences (forking a
sequence whose last block is partly filled is what makes the next append
copy-on-write).  The root stays alive and is never decoded.

This module only draws numbers: tail lengths, the pool size bound and which
ids retire / get forked.  The allocator decisions live elsewhere.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

from .configs import PrefixSharedConfig, blocks_for

# value streams (see workloads.values.draw_normal_storage)
STREAM_PREFIX_K = 2
STREAM_PREFIX_V = 3
STREAM_TAIL_K = 4
STREAM_TAIL_V = 5
STREAM_ITER_BASE = 100  # iteration t uses (seed, 100 + t, {1: q, 2: k, 3: v})
STREAM_CHURN_BASE = 100000


@dataclass(frozen=True)
class PrefixSharedPlan:
    tails: np.ndarray  # int64 [num_seqs]
    num_blocks: int
    free_order: np.ndarray  # int32 [num_blocks]


def pool_blocks_prefix_shared(cfg: PrefixSharedConfig, tails: np.ndarray) -> int:
    """1.25x an upper bound on blocks ever in use.

    Bound: the prefix blocks, every tail's blocks, at most ceil(T/16) new
    blocks per sequence ever decoding over T iterations (the initial ones
    plus every admitted one), and one copied block per admitted fork.
    """
    bs = cfg.block_size
    prefix = blocks_for(cfg.prefix_len, bs)
    tails_b = int(sum(blocks_for(t, bs) for t in tails))
    ever = cfg.num_seqs + cfg.iterations * cfg.churn
    growth = ever * blocks_for(cfg.iterations, bs) + cfg.iterations * cfg.churn
    return int(math.ceil(1.25 * (prefix + tails_b + growth)))


def draw_prefix_shared_plan(cfg: PrefixSharedConfig) -> PrefixSharedPlan:
    rng = np.random.default_rng(cfg.seed)
    tails = rng.integers(0, cfg.tail_max + 1, size=cfg.num_seqs).astype(np.int64)
    nb = pool_blocks_prefix_shared(cfg, tails)
    order = rng.permutation(nb).astype(np.int32)
    return PrefixSharedPlan(tails=tails, num_blocks=nb, free_order=order)


def choose_churn(cfg: PrefixSharedConfig, iteration: int,
                 live_ids: Sequence[int]) -> Tuple[List[int], List[int]]:
    """Seeded (retire ids ascending, fork parents in admission order)."""
    live = sorted(int(i) for i in live_ids)
    k = cfg.churn
    rng = np.random.default_rng((cfg.seed, STREAM_CHURN_BASE + int(iteration)))
    ridx = rng.choice(len(live), size=k, replace=False)
    retire = sorted(live[i] for i in ridx)
    rset = set(retire)
    survivors = [s for s in live if s not in rset]
    pidx = rng.choice(len(survivors), size=k, replace=False)
    parents = [survivors[i] for i in pidx]
    return retire, parents
