"""Pins of the chunked-prefill oracle (CPU).

The oracle's prefill is each chunk query decoded over its causal prefix.
It is pinned to things other than itself:
  * torch's scaled_dot_product_attention in float64 with an explicit
    boolean mask aligned to the end of the context, GQA by repeating KV
    heads;
  * closed forms: the first token of a prompt (empty cache) returns its own
    value row exactly; a chunk with q = 0 averages the V rows it can see;
  * a mask aligned to the start of the context (query t sees 0 .. t) gives
    different results once something is cached, so the alignment is
    checked, not assumed;
  * a pure-Python triple loop on a tiny case;
  * chunk invariance through the allocator and the mirrored pool: every
    prompt of a workload prefilled chunk by chunk gives the same outputs as
    the prompt attended densely in one piece, and the paged K/V gathered
    through the tables equal the dense rows bit for bit.
"""

import math

import numpy as np
import pytest
import torch

from oracle.attention import decode_attention, prefill_attention, storage_to_f64
from oracle.runs import PrefillRun
from workloads.prefill import (PREFILL_CONFIGS, draw_prefill_shapes, draw_prefill_values,
                               prefill_config_by_name, prompt_offsets)


def sdpa_prefill(q, K, V, scale):
    """torch SDPA (float64) over the dense context with the causal mask
    aligned to the end of the context."""
    T, Hq, d = q.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)  # [Hq][T][d]
    kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)
    vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)
    C = L - T
    pos_q = torch.arange(T)[:, None] + C
    pos_k = torch.arange(L)[None, :]
    mask = pos_k <= pos_q  # True = attend
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("C,T,Hq,Hkv,d", [(0, 1, 2, 2, 8), (0, 17, 4, 4, 16), (5, 9, 4, 2, 16),
                                          (40, 3, 8, 2, 32), (31, 33, 6, 3, 8), (100, 1, 4, 1, 16)])
def test_prefill_matches_sdpa_with_end_aligned_mask(C, T, Hq, Hkv, d):
    rng = np.random.default_rng(C * 1000 + T)
    q = rng.standard_normal((T, Hq, d))
    K = rng.standard_normal((C + T, Hkv, d))
    V = rng.standard_normal((C + T, Hkv, d))
    scale = 1 / math.sqrt(d)
    got = prefill_attention(q, K, V, scale)
    ref = sdpa_prefill(q, K, V, scale)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_start_aligned_mask_is_detected():
    rng = np.random.default_rng(3)
    C, T, H, d = 7, 5, 2, 8
    q = rng.standard_normal((T, H, d))
    K = rng.standard_normal((C + T, H, d))
    V = rng.standard_normal((C + T, H, d))
    got = prefill_attention(q, K, V, 0.3)
    wrong = np.stack([decode_attention(q[t], K[:t + 1], V[:t + 1], 0.3) for t in range(T)])
    assert np.max(np.abs(got - wrong)) > 1e-3


def test_closed_forms():
    rng = np.random.default_rng(5)
    T, Hq, Hkv, d = 6, 4, 2, 8
    q = rng.standard_normal((T, Hq, d))
    K = rng.standard_normal((T, Hkv, d))
    V = rng.standard_normal((T, Hkv, d))
    out = prefill_attention(q, K, V, 0.5)
    for h in range(Hq):
        assert np.array_equal(out[0, h], V[0, h // 2])  # empty cache: own value row
    z = prefill_attention(np.zeros_like(q), K, V, 0.5)
    for t in range(T):
        for h in range(Hq):
            assert np.allclose(z[t, h], V[:t + 1, h // 2].mean(axis=0), atol=1e-14)


def test_brute_force_triple_loop():
    rng = np.random.default_rng(9)
    C, T, Hq, Hkv, d = 3, 4, 4, 2, 3
    q = rng.standard_normal((T, Hq, d))
    K = rng.standard_normal((C + T, Hkv, d))
    V = rng.standard_normal((C + T, Hkv, d))
    scale = 0.7
    got = prefill_attention(q, K, V, scale)
    for t in range(T):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            n = C + t + 1
            s = [scale * sum(q[t, h, i] * K[j, g, i] for i in range(d)) for j in range(n)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = sum(w)
            for i in range(d):
                o = sum(w[j] * V[j, g, i] for j in range(n)) / z
                assert abs(got[t, h, i] - o) < 1e-12


def test_schedules_cover_every_token_once():
    for cfg in PREFILL_CONFIGS:
        sh = draw_prefill_shapes(cfg)
        seen = [0] * len(sh.prompts)
        for step in sh.steps:
            assert len({s for s, _, _ in step}) == len(step)
            for seq, t0, n in step:
                assert t0 == seen[seq] and 1 <= n <= cfg.chunk_tokens
                seen[seq] += n
        assert seen == [int(p) for p in sh.prompts]
        assert sorted(sh.free_order.tolist()) == list(range(sh.num_blocks))


@pytest.mark.parametrize("name", ["pf_tiny_f16", "pf_tiny_gqa_bf16"])
def test_chunked_run_equals_dense_prompt(name):
    cfg = prefill_config_by_name(name)
    sh = draw_prefill_shapes(cfg)
    vals = draw_prefill_values(cfg, sh.prompts)
    width = -(-int(sh.prompts.max()) // 16)
    run = PrefillRun(cfg, sh, width, vals)
    q, k, v = (storage_to_f64(x, cfg.dtype) for x in vals)
    row0 = prompt_offsets(sh.prompts)
    got = {i: [] for i in range(len(sh.prompts))}
    for _ in sh.steps:
        for seq, t0, n, slots in run.append_step():
            got[seq].append(run.attend(seq, t0, n))
            # paged view == dense rows, bit for bit
            Kp, Vp = run.mirror.gather(run.alloc.table(seq), t0 + n)
            r = int(row0[seq])
            assert np.array_equal(Kp, vals[1][r:r + t0 + n])
            assert np.array_equal(Vp, vals[2][r:r + t0 + n])
    for i, P in enumerate(sh.prompts):
        r = int(row0[i])
        dense = prefill_attention(q[r:r + P], k[r:r + P], v[r:r + P], cfg.scale)
        assert np.max(np.abs(np.concatenate(got[i]) - dense)) < 1e-12
        assert len(run.alloc.table(i)) == -(-int(P) // 16)


def test_sampled_rows_match_full_chunk():
    cfg = prefill_config_by_name("pf_tiny_f16")
    sh = draw_prefill_shapes(cfg)
    vals = draw_prefill_values(cfg, sh.prompts)
    run = PrefillRun(cfg, sh, 8, vals)
    run.append_step()
    items = run.append_step()
    seq, t0, n, _ = items[0]
    full = run.attend(seq, t0, n)
    rows = [0, n // 2, n - 1]
    assert np.array_equal(run.attend(seq, t0, n, rows=rows), full[rows])
