"""Seeded synthetic workloads for chunked paged prefill.

The lesson on continuous batching ("PagedAttention e continuous batching",
01 · Conceito, the paragraph on the scheduler) says that a scheduler mixes
prefill and decode work and often slices a long prefill so that a
newcomer's 30,000-token prompt does not stall everybody's next token.  It
gives no other size.  The workloads below are readings of that sentence:

  * ``pf_tiny_f16``, ``pf_tiny_gqa_bf16``: a few short prompts cut into
    small chunks (parity at sizes the oracle finishes in seconds, ragged
    chunk tails, several chunks per prompt, grouped-query heads);
  * ``pf_long_f16``: the newcomer itself, one 30,000-token prompt sliced
    into 2048-token chunks, with the GPT-style heads of the tutorial
    (32 x 128, fp16);
  * ``pf_batch_bf16``: sixteen prompts of U[512, 4096] tokens prefilled
    together in 1024-token slices, with the long-context workload's
    grouped-query heads (32 query / 8 KV, bf16);
  * ``pf_slice_f16``: the same 30,000-token newcomer in 256-token slices,
    the thin slices a scheduler takes when it guards the decoding
    sequences' next token (each launch is then a few tiles deep in a long
    context).

Schedule: step k takes, from every prompt that still has tokens left, its
next ``min(chunk, remaining)`` tokens; the first chunk allocates the
sequence, later chunks append.  Sequence i has id i.  Values: q, k and v of
every prompt token are drawn in (sequence, token) order from streams 1, 2
and 3 of ``workloads.values.draw_normal_storage``.  This module draws
numbers only.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Tuple

import numpy as np

from .configs import BLOCK_SIZE, blocks_for
from .values import draw_normal_storage


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    index: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    chunk_tokens: int
    fixed_prompts: Tuple[int, ...] = ()
    num_seqs: int = 0
    prompt_lo: int = 0
    prompt_hi: int = 0
    block_size: int = BLOCK_SIZE
    description: str = ""

    @property
    def seed(self) -> int:
        return 42 + self.index

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


PREFILL_CONFIGS = (
    PrefillConfig(name="pf_tiny_f16", index=10, dtype="f16", num_q_heads=4, num_kv_heads=4,
                  head_dim=64, chunk_tokens=32, fixed_prompts=(37, 70, 9),
                  description="3 short prompts in 32-token chunks, MHA, d=64"),
    PrefillConfig(name="pf_tiny_gqa_bf16", index=11, dtype="bf16", num_q_heads=8, num_kv_heads=2,
                  head_dim=128, chunk_tokens=16, fixed_prompts=(50, 23, 1),
                  description="3 short prompts in 16-token chunks, GQA 8/2, d=128"),
    PrefillConfig(name="pf_long_f16", index=12, dtype="f16", num_q_heads=32, num_kv_heads=32,
                  head_dim=128, chunk_tokens=2048, fixed_prompts=(30000,),
                  description="one 30,000-token prompt sliced into 2048-token chunks"),
    PrefillConfig(name="pf_batch_bf16", index=13, dtype="bf16", num_q_heads=32, num_kv_heads=8,
                  head_dim=128, chunk_tokens=1024, num_seqs=16, prompt_lo=512, prompt_hi=4096,
                  description="16 prompts of U[512, 4096] tokens in 1024-token slices, GQA 32/8"),
    PrefillConfig(name="pf_slice_f16", index=14, dtype="f16", num_q_heads=32, num_kv_heads=32,
                  head_dim=128, chunk_tokens=256, fixed_prompts=(30000,),
                  description="one 30,000-token prompt in 256-token slices"),
)


def prefill_config_by_name(name: str) -> PrefillConfig:
    for c in PREFILL_CONFIGS:
        if c.name == name:
            return c
    raise KeyError(f"unknown prefill workload {name!r}")


@dataclass(frozen=True)
class PrefillShapes:
    prompts: np.ndarray          # int64 [B]
    num_blocks: int
    free_order: np.ndarray       # int32 [num_blocks]
    steps: List[List[Tuple[int, int, int]]]  # per step: (seq, first token, tokens)


def draw_prefill_shapes(cfg: PrefillConfig) -> PrefillShapes:
    rng = np.random.default_rng(cfg.seed)
    if cfg.fixed_prompts:
        prompts = np.asarray(cfg.fixed_prompts, dtype=np.int64)
    else:
        prompts = rng.integers(cfg.prompt_lo, cfg.prompt_hi + 1, size=cfg.num_seqs).astype(np.int64)
    need = int(sum(blocks_for(int(p), cfg.block_size) for p in prompts))
    nb = int(math.ceil(1.25 * need))
    order = rng.permutation(nb).astype(np.int32)
    steps: List[List[Tuple[int, int, int]]] = []
    done = [0] * len(prompts)
    while any(done[i] < prompts[i] for i in range(len(prompts))):
        step = []
        for i, p in enumerate(prompts):
            n = min(cfg.chunk_tokens, int(p) - done[i])
            if n > 0:
                step.append((i, done[i], n))
                done[i] += n
        steps.append(step)
    return PrefillShapes(prompts=prompts, num_blocks=nb, free_order=order, steps=steps)


def draw_prefill_values(cfg: PrefillConfig, prompts: np.ndarray):
    """q [sum P][H_q][d], k and v [sum P][H_kv][d] storage bits, rows in
    (sequence, token) order."""
    n = int(np.sum(prompts))
    q = draw_normal_storage((cfg.seed, 1), (n, cfg.num_q_heads, cfg.head_dim), cfg.dtype)
    k = draw_normal_storage((cfg.seed, 2), (n, cfg.num_kv_heads, cfg.head_dim), cfg.dtype)
    v = draw_normal_storage((cfg.seed, 3), (n, cfg.num_kv_heads, cfg.head_dim), cfg.dtype)
    return q, k, v


def prompt_offsets(prompts: np.ndarray) -> np.ndarray:
    """Row of token 0 of each prompt in the value arrays."""
    return np.concatenate([[0], np.cumsum(prompts)[:-1]]).astype(np.int64)
