"""Pins for oracle/attention.py (CPU).

The oracle's attention is pinned to things other than itself:
  * torch's scaled_dot_product_attention (a library routine for dense
    attention) run in float64 on the dense, never-paged shadow cache -- the
    pages state that paging leaves the dense result unchanged;
  * closed forms: a one-token context returns that token's value row; a zero
    query or identical keys return the mean of the value rows; one dominant
    logit returns its row; adding a constant row to V shifts the output by it;
  * grouped-query head mapping against SDPA on explicitly repeated KV heads;
  * the split-K combine against the unsplit result;
  * bf16 / fp16 bit decoding against the formats' definitions.
"""

import math

import numpy as np
import pytest
import torch

from oracle.attention import (combine_partials, decode_attention, decode_partials,
                              storage_to_f64)
from oracle.kvcache import DenseShadow
from oracle.runs import DecodeRun
from workloads import config_by_name, draw_decode_values
from workloads.configs import draw_decode_shapes


def sdpa64(q, K, V, scale):
    """torch SDPA in float64; q [Hq][d], K/V [L][Hkv][d] -> [Hq][d]."""
    Hq = q.shape[0]
    Hkv = K.shape[1]
    G = Hq // Hkv
    qt = torch.from_numpy(q)[None, :, None, :]  # [1, Hq, 1, d]
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt.contiguous(), Vt.contiguous(),
                                                         scale=scale)
    return o[0, :, 0, :].numpy()


def tiny_run():
    cfg = config_by_name("tiny_f32")
    sh = draw_decode_shapes(cfg)
    vals = draw_decode_values(cfg, sh.lens)
    q, k, v = vals["q"], vals["k"], vals["v"]
    run = DecodeRun(cfg, sh.lens, sh.num_blocks, sh.free_order, 8)
    run.write_context(k, v)
    return cfg, sh, q, k, v, run


def test_paged_oracle_matches_library_sdpa_on_dense_shadow():
    cfg, sh, q, k, v, run = tiny_run()
    shadow = DenseShadow(cfg.num_kv_heads, cfg.head_dim, np.float32)
    off = 0
    for i, L in enumerate(sh.lens):
        shadow.new(i)
        shadow.append(i, k[off:off + L], v[off:off + L])
        off += L
    for i in range(cfg.num_seqs):
        got = run.attend(i, q[i])
        Kd, Vd = shadow.get(i)
        want = sdpa64(q[i].astype(np.float64), Kd.astype(np.float64), Vd.astype(np.float64),
                      cfg.scale)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_single_token_context_returns_its_value_row():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((4, 64))
    K = rng.standard_normal((1, 4, 64))
    V = rng.standard_normal((1, 4, 64))
    out = decode_attention(q, K, V, 0.125)
    assert np.array_equal(out, V[0])


@pytest.mark.parametrize("L", [2, 17, 60])
def test_zero_query_and_equal_keys_give_mean_of_values(L):
    rng = np.random.default_rng(L)
    V = rng.standard_normal((L, 2, 32))
    K = rng.standard_normal((L, 2, 32))
    q0 = np.zeros((2, 32))
    np.testing.assert_allclose(decode_attention(q0, K, V, 0.3), V.mean(axis=0), atol=1e-14)
    Keq = np.repeat(rng.standard_normal((1, 2, 32)), L, axis=0)
    q = rng.standard_normal((2, 32))
    np.testing.assert_allclose(decode_attention(q, Keq, V, 0.3), V.mean(axis=0), atol=1e-13)


def test_dominant_logit_selects_its_row():
    rng = np.random.default_rng(5)
    L, d = 33, 16
    K = rng.standard_normal((L, 1, d)) * 0.01
    V = rng.standard_normal((L, 1, d))
    q = np.zeros((1, d))
    q[0, 3] = 1.0
    K[20, 0, 3] = 1000.0
    out = decode_attention(q, K, V, 1.0)
    np.testing.assert_allclose(out[0], V[20, 0], atol=1e-12)


def test_softmax_weights_sum_to_one_value_shift():
    rng = np.random.default_rng(6)
    L, d = 45, 64
    q = rng.standard_normal((4, d))
    K = rng.standard_normal((L, 4, d))
    V = rng.standard_normal((L, 4, d))
    c = rng.standard_normal((4, d))
    base = decode_attention(q, K, V, 1 / 8)
    shifted = decode_attention(q, K, V + c[None], 1 / 8)
    np.testing.assert_allclose(shifted, base + c, atol=1e-12)


def test_scale_enters_as_scaled_query():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((2, 16))
    K = rng.standard_normal((9, 2, 16))
    V = rng.standard_normal((9, 2, 16))
    np.testing.assert_allclose(decode_attention(q, K, V, 0.5), decode_attention(0.5 * q, K, V, 1.0),
                               atol=1e-14)


def test_token_order_does_not_matter():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((2, 16))
    K = rng.standard_normal((21, 2, 16))
    V = rng.standard_normal((21, 2, 16))
    perm = rng.permutation(21)
    np.testing.assert_allclose(decode_attention(q, K, V, 0.25), decode_attention(q, K[perm], V[perm], 0.25),
                               atol=1e-13)


def test_gqa_head_mapping_matches_sdpa_with_repeated_kv_heads():
    rng = np.random.default_rng(9)
    Hq, Hkv, d, L = 32, 8, 128, 70
    q = rng.standard_normal((Hq, d))
    K = rng.standard_normal((L, Hkv, d))
    V = rng.standard_normal((L, Hkv, d))
    scale = 1 / math.sqrt(d)
    got = decode_attention(q, K, V, scale)
    np.testing.assert_allclose(got, sdpa64(q, K, V, scale), atol=1e-12)
    # a wrong grouping (h % Hkv) must differ: the pin can tell them apart
    Kperm = K[:, [h % Hkv for h in range(Hq)], :]
    Vperm = V[:, [h % Hkv for h in range(Hq)], :]
    wrong = np.stack([decode_attention(q[h:h + 1], Kperm[:, h:h + 1], Vperm[:, h:h + 1], scale)[0]
                      for h in range(Hq)])
    assert np.abs(wrong - got).max() > 1e-3


@pytest.mark.parametrize("P", [16, 32, 48, 512, 4096])
def test_split_k_combine_equals_unsplit(P):
    rng = np.random.default_rng(P)
    L, Hq, Hkv, d = 1000, 8, 2, 64
    q = rng.standard_normal((Hq, d))
    K = rng.standard_normal((L, Hkv, d))
    V = rng.standard_normal((L, Hkv, d))
    m, l_, o = decode_partials(q, K, V, 0.125, P)
    assert m.shape[0] == -(-L // P)
    np.testing.assert_allclose(combine_partials(m, l_, o), decode_attention(q, K, V, 0.125),
                               atol=1e-12)


def test_storage_decoding_matches_format_definitions():
    bf = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    want = [1.0, -2.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, -0.0]
    got = storage_to_f64(bf, "bf16")
    assert list(got) == want
    assert np.signbit(got[4])
    h = np.array([0x3C00, 0xC000, 0x0001, 0x7BFF], dtype=np.uint16).view(np.float16)
    assert list(storage_to_f64(h, "f16")) == [1.0, -2.0, 2.0 ** -24, 65504.0]
    f = np.array([1.5, -3.25], dtype=np.float32)
    assert list(storage_to_f64(f, "f32")) == [1.5, -3.25]
