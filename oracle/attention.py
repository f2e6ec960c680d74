"""fp64 decode attention over paged K/V (oracle; test infrastructure only).

The pages never print the attention formula; they fix two facts about it:
the attention kernel reads keys and values by following each sequence's
block table ([lesson] paragraph 3; [preview] "La idea de PagedAttention",
step 5), and paging leaves the FLOPs and the result of dense attention
unchanged ([preview] "Lo que deberías llevarte", item 2).  So the result is
dense scaled dot-product attention over the sequence's logical tokens,
computed here in float64:

    s_j = scale * <q_h, k_{j, g(h)}>,  p = exp(s - max s),
    o_h = sum_j p_j v_{j, g(h)} / sum_j p_j,

with scale = 1/sqrt(d) and, reading for grouped-query attention,
g(h) = h // (H_q / H_kv) (contiguous groups of query heads share a KV head).

Chunked prefill: a chunk of T new tokens appended after C cached ones
(L = C + T) brings T queries; the query of chunk token t sits at position
C + t and attends to positions 0 .. C + t of the same sequence, its own
key included.  The lesson names the slicing of long prefills into chunks
("PagedAttention e continuous batching", 01 · Conceito, the paragraph on
the scheduler) without printing a mask; the causal reading is the plain
one (a prompt token never sees later tokens, so slicing a prompt does not
change any output).

Split-K: a sequence's tokens cut into partitions of P tokens give per-
partition (m_p, l_p, o~_p) = (max s, sum exp(s - m_p), sum exp(s - m_p) v);
the exact combine is  o = sum_p e^{m_p - M} o~_p / sum_p e^{m_p - M} l_p
with M = max_p m_p.  The partition size is a property of the workload, not
of the pages.
"""

from __future__ import annotations

import numpy as np


def storage_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of storage-dtype bits (bf16 via its top 16 bits)."""
    a = np.asarray(bits)
    if dtype == "f32":
        return a.astype(np.float32, copy=False).astype(np.float64)
    if dtype == "f16":
        return a.astype(np.float16, copy=False).astype(np.float64)
    if dtype == "bf16":
        u = a.astype(np.uint16, copy=False).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def _kv_head(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    group = num_q_heads // num_kv_heads
    return h // group


def decode_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """One query token per head.

    q: [H_q][d] float64;  K, V: [L][H_kv][d] float64 (L >= 1)  ->  [H_q][d].
    """
    Hq, d = q.shape
    L, Hkv, _ = K.shape
    if L < 1:
        raise ValueError("attention over an empty context is undefined")
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    out = np.empty((Hq, d), dtype=np.float64)
    for h in range(Hq):
        g = _kv_head(h, Hq, Hkv)
        s = scale * (K[:, g, :] @ q[h])  # [L]
        m = np.max(s)
        p = np.exp(s - m)
        out[h] = (p @ V[:, g, :]) / np.sum(p)
    return out


def prefill_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """The queries of the last T tokens of a sequence, causally.

    q: [T][H_q][d] float64 (the chunk's queries, in token order);
    K, V: [L][H_kv][d] float64, the whole context including the chunk
    (L >= T)  ->  [T][H_q][d].  Query t attends to K/V rows 0 .. L - T + t.
    """
    T = q.shape[0]
    L = K.shape[0]
    if T > L:
        raise ValueError("the chunk is longer than the context")
    C = L - T
    out = np.empty(q.shape, dtype=np.float64)
    for t in range(T):
        out[t] = decode_attention(q[t], K[:C + t + 1], V[:C + t + 1], scale)
    return out


def decode_partials(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                    partition_tokens: int):
    """Per-partition (m [P][H_q], l [P][H_q], o~ [P][H_q][d]) in float64."""
    Hq, d = q.shape
    L, Hkv, _ = K.shape
    nparts = -(-L // partition_tokens)
    m = np.empty((nparts, Hq))
    l_ = np.empty((nparts, Hq))
    o = np.empty((nparts, Hq, d))
    for p_ in range(nparts):
        lo, hi = p_ * partition_tokens, min(L, (p_ + 1) * partition_tokens)
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            s = scale * (K[lo:hi, g, :] @ q[h])
            m[p_, h] = np.max(s)
            e = np.exp(s - m[p_, h])
            l_[p_, h] = np.sum(e)
            o[p_, h] = e @ V[lo:hi, g, :]
    return m, l_, o


def combine_partials(m: np.ndarray, l_: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Exact combine of split-K partials -> [H_q][d]."""
    M = np.max(m, axis=0)  # [H_q]
    w = np.exp(m - M[None, :])  # [P][H_q]
    num = np.sum(w[:, :, None] * o, axis=0)
    den = np.sum(w * l_, axis=0)
    return num / den[:, None]
