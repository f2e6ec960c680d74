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


def draw_churn(cfg: PrefixSharedConfig, iteration: int, n_live: int) -> Tuple[np.ndarray, np.ndarray]:
    """Iteration's seeded draws for ``n_live`` decoding sequences: positions
    (in ascending id order) of the ``churn`` that retire, then positions
    among the survivors of the ``churn`` fork parents."""
    k = cfg.churn
    rng = np.random.default_rng((cfg.seed, STREAM_CHURN_BASE + int(iteration)))
    ridx = rng.choice(n_live, size=k, replace=False)
    pidx = rng.choice(n_live - k, size=k, replace=False)
    return ridx, pidx


def apply_churn(live_ids: Sequence[int], ridx: np.ndarray, pidx: np.ndarray) -> Tuple[List[int], List[int]]:
    """(retire ids ascending, fork parents in admission order) for the draws."""
    live = np.sort(np.asarray(live_ids, dtype=np.int64))
    retire = np.sort(live[ridx])
    survivors = np.delete(live, ridx)  # ids are distinct: ascending order kept
    return retire.tolist(), survivors[pidx].tolist()


def choose_churn(cfg: PrefixSharedConfig, iteration: int,
                 live_ids: Sequence[int]) -> Tuple[List[int], List[int]]:
    """Seeded (retire ids ascending, fork parents in admission order)."""
    ridx, pidx = draw_churn(cfg, iteration, len(live_ids))
    return apply_churn(live_ids, ridx, pidx)
