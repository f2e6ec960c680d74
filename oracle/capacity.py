"""Capacity arithmetic printed on the pages (oracle; test infrastructure).

Each helper restates a count the pages use; the tests pin them to the
numbers the pages print (``tests/golden/pages_capacity.json``).
"""

from __future__ import annotations

import math


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V (the factor 2) for every layer, KV head and head dim.

    [tutorial] "Configurando as Constantes": GPT-style 32 x 32 x 128 in fp16.
    """
    return 2 * layers * kv_heads * head_dim * elem_bytes


def blocks_for_tokens(n_tokens: int, block_size: int) -> int:
    """Blocks a sequence of n tokens holds ([preview] step 3)."""
    return -(-n_tokens // block_size)


def tail_waste_slots(n_tokens: int, block_size: int) -> int:
    """Unused rows of the last block ([preview] "Propiedades": < block)."""
    return block_size * blocks_for_tokens(n_tokens, block_size) - n_tokens


def sessions_that_fit(pool_bytes: float, bytes_per_session: float) -> int:
    """Whole sessions a state pool holds ([lesson] paragraphs 2 and 4)."""
    return int(math.floor(pool_bytes / bytes_per_session))


def dense_waste_fraction(mean_len: float, max_len: float) -> float:
    """Share of a max-length reservation left unused ([preview] Problema 1)."""
    return 1.0 - mean_len / max_len


def padding_factor(padded_len: float, actual_len: float) -> float:
    """Work inflation of padding a sequence to the batch max ([preview] Problema 3)."""
    return padded_len / actual_len


def utilisation_gap(lengths, max_len: int, block_size: int) -> dict:
    """Naive contiguous reservation vs paged blocks for one set of
    concurrent requests ([tutorial] opening paragraph and "Cache KV
    Ingenuo": every request reserves max_len tokens up front; paging holds
    ceil(L / block) blocks per request, [preview] steps 1-3).  Token counts;
    multiply by the bytes per token for memory."""
    used = sum(int(x) for x in lengths)
    naive = len(lengths) * int(max_len)
    blocks = sum(blocks_for_tokens(int(x), block_size) for x in lengths)
    paged = blocks * block_size
    return {"requests": len(lengths), "tokens_used": used, "naive_reserved_tokens": naive,
            "paged_blocks": blocks, "paged_reserved_tokens": paged,
            "naive_waste_tokens": naive - used, "paged_waste_tokens": paged - used}
