"""The five synthetic paged-decode workloads and their seeded shape draws.

Each workload is a frozen dataclass.  Shapes and the seeded draws follow
the workload descriptions the method is measured on (block size 16,
GPT-style 32 heads x 128 dims in fp16, a ragged log-uniform batch, ten
32,768-token GQA sessions, and a prefix-shared continuous-batching loop).
The tutorial these shapes come from ("Paged Attention em Large Language
Models LLMs", section "Configurando as Constantes") fixes 32 heads, head
dim 128, fp16, 16 tokens per page, a 2048-token maximum, a mean response
of 500 tokens and seed 42; workload ``k`` (0-based) is seeded with
``42 + k``.

Integerisation rules (the workload text gives distributions, not integer
rules):
  * exponential lengths: ``clip(ceil(x), 1, max_len)``;
  * log-uniform lengths: ``clip(round(exp(u)), lo, hi)`` with
    ``u ~ U(ln lo, ln hi)``, then the pinned lengths overwrite distinct
    seeded positions;
  * pool size where not given: ``ceil(1.25 * sum(ceil(L_i / 16)))``.

Random stream layout (so that any part can be regenerated alone):
``numpy.random.default_rng(seed)`` draws the lengths and then the free-block
permutation; values come from ``default_rng((seed, stream, chunk))`` in
``workloads.values``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

BLOCK_SIZE = 16


@dataclass(frozen=True)
class DecodeConfig:
    """One decode batch: B sequences, one query token each."""

    name: str
    index: int
    dtype: str  # "f32" | "f16" | "bf16"
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    length_rule: str  # "fixed" | "exponential" | "loguniform" | "constant"
    block_size: int = BLOCK_SIZE
    fixed_lengths: Tuple[int, ...] = ()
    mean_len: float = 0.0
    min_len: int = 1
    max_len: int = 0
    pinned_lengths: Tuple[int, ...] = ()
    pool_blocks: int = 0  # 0 -> 1.25x the blocks needed
    partition_tokens: int = 0  # 0 -> library default
    description: str = ""

    @property
    def seed(self) -> int:
        return 42 + self.index

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


@dataclass(frozen=True)
class PrefixSharedConfig:
    """Continuous-batching loop over sequences sharing one prompt prefix."""

    name: str
    index: int
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    prefix_len: int
    tail_max: int
    iterations: int
    retire_frac: float
    block_size: int = BLOCK_SIZE
    description: str = ""

    @property
    def seed(self) -> int:
        return 42 + self.index

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def churn(self) -> int:
        """Sequences retired (and admitted) per iteration: round(5% of B)."""
        return int(round(self.retire_frac * self.num_seqs))


CONFIGS = (
    DecodeConfig(
        name="tiny_f32", index=0, dtype="f32", num_seqs=4, num_q_heads=4,
        num_kv_heads=4, head_dim=64, length_rule="fixed",
        fixed_lengths=(5, 17, 33, 60), pool_blocks=32,
        description="tiny single-layer fp32 decode, 4 seqs, pool of 32 blocks"),
    DecodeConfig(
        name="gpt_f16", index=1, dtype="f16", num_seqs=64, num_q_heads=32,
        num_kv_heads=32, head_dim=128, length_rule="exponential",
        mean_len=500.0, min_len=1, max_len=2048,
        description="GPT-style fp16 decode batch, 64 seqs, L ~ Exp(500) in [1,2048]"),
    DecodeConfig(
        name="ragged_bf16", index=2, dtype="bf16", num_seqs=96, num_q_heads=32,
        num_kv_heads=32, head_dim=128, length_rule="loguniform",
        min_len=5, max_len=10000, pinned_lengths=(60, 200, 1500),
        description="high-variance ragged bf16 batch, 96 seqs, log-uniform [5,10000]"),
    DecodeConfig(
        name="gqa_long_bf16", index=3, dtype="bf16", num_seqs=10, num_q_heads=32,
        num_kv_heads=8, head_dim=128, length_rule="constant", max_len=32768,
        partition_tokens=512,
        description="long-context GQA bf16, 10 x 32768 tokens, 32 q / 8 kv heads"),
)

PREFIX_SHARED = PrefixSharedConfig(
    name="prefix_shared_f16", index=4, dtype="f16", num_seqs=256, num_q_heads=32,
    num_kv_heads=32, head_dim=128, prefix_len=4096, tail_max=1024, iterations=64,
    retire_frac=0.05,
    description="256 seqs sharing a 4096-token prefix, 64 continuous-batching iterations")

ALL_CONFIGS = CONFIGS + (PREFIX_SHARED,)


def config_by_name(name: str):
    for c in ALL_CONFIGS:
        if c.name == name:
            return c
    raise KeyError(f"unknown workload {name!r}; known: {[c.name for c in ALL_CONFIGS]}")


def blocks_for(n_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """Number of blocks that hold n tokens (a count used to size pools)."""
    return -(-int(n_tokens) // block_size)


def draw_context_lengths(cfg: DecodeConfig, rng: Optional[np.random.Generator] = None) -> np.ndarray:
    """Seeded context lengths (int64 array of B), first draw of the shape stream."""
    if rng is None:
        rng = np.random.default_rng(cfg.seed)
    B = cfg.num_seqs
    if cfg.length_rule == "fixed":
        lens = np.asarray(cfg.fixed_lengths, dtype=np.int64)
    elif cfg.length_rule == "constant":
        lens = np.full(B, cfg.max_len, dtype=np.int64)
    elif cfg.length_rule == "exponential":
        x = rng.exponential(cfg.mean_len, size=B)
        lens = np.clip(np.ceil(x), cfg.min_len, cfg.max_len).astype(np.int64)
    elif cfg.length_rule == "loguniform":
        u = rng.uniform(math.log(cfg.min_len), math.log(cfg.max_len), size=B)
        lens = np.clip(np.round(np.exp(u)), cfg.min_len, cfg.max_len).astype(np.int64)
        pos = rng.choice(B, size=len(cfg.pinned_lengths), replace=False)
        lens[pos] = np.asarray(cfg.pinned_lengths, dtype=np.int64)
    else:
        raise ValueError(cfg.length_rule)
    assert lens.shape == (B,)
    return lens


def pool_blocks_for(cfg: DecodeConfig, lens: np.ndarray) -> int:
    if cfg.pool_blocks:
        return int(cfg.pool_blocks)
    need = int(sum(blocks_for(L, cfg.block_size) for L in lens))
    return int(math.ceil(1.25 * need))


def draw_free_order(num_blocks: int, rng: np.random.Generator) -> np.ndarray:
    """Seeded permutation of the physical block ids (int32)."""
    return rng.permutation(num_blocks).astype(np.int32)


@dataclass(frozen=True)
class DecodeShapes:
    lens: np.ndarray
    num_blocks: int
    free_order: np.ndarray
    extra: dict = field(default_factory=dict)


def draw_decode_shapes(cfg: DecodeConfig) -> DecodeShapes:
    """Lengths, pool size and free order for a decode workload, in stream order."""
    rng = np.random.default_rng(cfg.seed)
    lens = draw_context_lengths(cfg, rng)
    nb = pool_blocks_for(cfg, lens)
    order = draw_free_order(nb, rng)
    return DecodeShapes(lens=lens, num_blocks=nb, free_order=order)
