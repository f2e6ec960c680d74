"""Seeded request lengths for the naive-vs-paged utilisation comparison.

The tutorial ("Paged Attention em Large Language Models LLMs") seeds its
simulation with 42, takes a mean response of 500 tokens and a 2048-token
maximum, and compares the two allocators at 10 to 200 concurrent requests.
Reading: request lengths are exponential with that mean, integerised as in
the decode workloads (``clip(ceil(x), 1, max_len)``); the batch of N
requests draws from ``default_rng((42, N))``.  Numbers only.
"""

from __future__ import annotations

import numpy as np

SEED = 42
MEAN_RESPONSE = 500
MAX_SEQ_LEN = 2048
BATCH_SIZES = (10, 20, 50, 100, 150, 200)


def draw_request_lengths(n: int, seed: int = SEED, mean: float = MEAN_RESPONSE,
                         max_len: int = MAX_SEQ_LEN) -> np.ndarray:
    rng = np.random.default_rng((seed, int(n)))
    x = rng.exponential(mean, size=int(n))
    return np.clip(np.ceil(x), 1, max_len).astype(np.int32)
