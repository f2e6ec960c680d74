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


def draw_request_trace(n: int, seed: int, rate: float = 4.0, prompt_lo: int = 16,
                       prompt_hi: int = 4096, mean_output: float = MEAN_RESPONSE,
                       max_output: int = MAX_SEQ_LEN, n_prefixes: int = 3, prefix_len: int = 512,
                       prefix_share: float = 0.3, n_classes: int = 2):
    """A seeded request stream for the scheduler: Poisson arrivals (``rate``
    per iteration), log-uniform prompt lengths, exponential output lengths
    (the tutorial's mean response), a seeded class per request, and a share
    of requests that start with one of a few shared prompt prefixes.
    Returns a list of dicts with the pkv_request fields."""
    rng = np.random.default_rng((seed, 7))
    gaps = rng.exponential(1.0 / rate, size=n)
    arrivals = np.floor(np.cumsum(gaps)).astype(np.int64)
    prompts = np.clip(np.round(np.exp(rng.uniform(np.log(prompt_lo), np.log(prompt_hi), size=n))),
                      prompt_lo, prompt_hi).astype(np.int64)
    outputs = np.clip(np.ceil(rng.exponential(mean_output, size=n)), 1, max_output).astype(np.int64)
    classes = rng.integers(0, n_classes, size=n)
    shared = rng.random(n) < prefix_share
    pid = rng.integers(0, n_prefixes, size=n)
    out = []
    for i in range(n):
        p_id, p_len, prompt = -1, 0, int(prompts[i])
        if shared[i] and n_prefixes > 0:
            p_id, p_len = int(pid[i]), prefix_len
            prompt = max(prompt, prefix_len + 1)
        out.append(dict(arrival=int(arrivals[i]), prompt_len=prompt, output_len=int(outputs[i]),
                        klass=int(classes[i]), prefix_id=p_id, prefix_len=p_len))
    return out
