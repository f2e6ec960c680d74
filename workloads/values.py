"""Seeded N(0,1) values in a storage dtype.

Values are drawn in float32 from ``numpy.random.default_rng((seed, stream,
chunk))`` in fixed chunks of ``CHUNK`` elements, so the result does not
depend on how many threads draw it, and any sub-range can be regenerated
alone.  They are then rounded to the storage type with round-to-nearest-
even: fp16 through numpy's own cast, bf16 by rounding the float32 bit
pattern to its upper 16 bits.  The storage arrays carry the exact bits
both sides read: ``float32``, ``float16``, or ``uint16`` for bf16.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Sequence

import numpy as np

CHUNK = 1 << 22

STORAGE_NUMPY = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


def storage_from_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype (round-to-nearest-even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        u = x.view(np.uint32)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
        return r.astype(np.uint16)
    raise ValueError(dtype)


def _draw_chunk(seed: Sequence[int], chunk: int, n: int, dtype: str) -> np.ndarray:
    rng = np.random.default_rng(tuple(int(s) for s in seed) + (int(chunk),))
    return storage_from_f32(rng.standard_normal(n, dtype=np.float32), dtype)


def draw_normal_storage(seed: Sequence[int], shape, dtype: str, threads: int = 0) -> np.ndarray:
    """N(0,1) values of ``shape`` in the storage dtype for stream ``seed``."""
    shape = tuple(int(s) for s in (shape if isinstance(shape, (tuple, list)) else (shape,)))
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=STORAGE_NUMPY[dtype])
    nchunks = -(-n // CHUNK) if n else 0
    if threads <= 0:
        threads = min(16, os.cpu_count() or 1)

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        out[lo:hi] = _draw_chunk(seed, c, hi - lo, dtype)

    if nchunks <= 1 or threads == 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


# value streams of a decode batch: q, then the context K and V rows in
# sequence order (sequence 0's L_0 rows first).
STREAM_Q, STREAM_K, STREAM_V = 1, 2, 3


def draw_decode_values(cfg, lens, which: str = "qkv"):
    """Storage-dtype q [B][H_q][d], k / v [sum L][H_kv][d] for a decode batch."""
    T = int(sum(int(x) for x in lens))
    out = {}
    if "q" in which:
        out["q"] = draw_normal_storage((cfg.seed, STREAM_Q),
                                       (cfg.num_seqs, cfg.num_q_heads, cfg.head_dim), cfg.dtype)
    if "k" in which:
        out["k"] = draw_normal_storage((cfg.seed, STREAM_K), (T, cfg.num_kv_heads, cfg.head_dim), cfg.dtype)
    if "v" in which:
        out["v"] = draw_normal_storage((cfg.seed, STREAM_V), (T, cfg.num_kv_heads, cfg.head_dim), cfg.dtype)
    return out
