"""Pins for oracle/capacity.py against the numbers the pages print (CPU)."""

import json
import math
import os

import pytest

from oracle import capacity as cap

KiB, MiB, GiB = 1 << 10, 1 << 20, 1 << 30


@pytest.fixture(scope="module")
def pages(golden_dir):
    with open(os.path.join(golden_dir, "pages_capacity.json")) as f:
        return json.load(f)


def test_gpt_style_bytes_per_token(pages):
    g = pages["gpt_kv_bytes_per_token"]
    assert cap.kv_bytes_per_token(g["layers"], g["heads"], g["head_dim"], g["elem_bytes"]) == g["value"]
    assert g["value"] == 512 * KiB


def test_qwen_like_reservation_and_blocks(pages):
    per_tok = pages["qwen_kv_bytes_per_token"]["value"]
    # 16 full-attention layers at 4 KiB each: 8 KV heads x 128 dims in bf16 is one such split
    assert cap.kv_bytes_per_token(16, 8, 128, 2) == per_tok
    r = pages["qwen_max_reservation_bytes"]
    assert per_tok * r["tokens"] == r["value"] == 16 * GiB
    b = pages["qwen_block_bytes"]
    assert b["block_tokens"] * per_tok == b["value"] == MiB


def test_qwen_sessions(pages):
    per_tok = pages["qwen_kv_bytes_per_token"]["value"]
    s = pages["qwen_session_kv_bytes"]
    assert s["tokens"] * per_tok == s["value"] == 2 * GiB
    tot = pages["qwen_session_total_mib"]
    assert s["value"] // MiB + tot["deltanet_state_mib"] == tot["value"]
    pool_mib = pages["qwen_state_pool_gib"]["mib"]
    assert round(pool_mib / 1024, 1) == pages["qwen_state_pool_gib"]["value"]
    assert cap.sessions_that_fit(pool_mib, tot["value"]) == pages["qwen_paged_sessions"]["value"]
    assert cap.sessions_that_fit(pool_mib * MiB, pages["qwen_max_reservation_bytes"]["value"]) == \
        pages["qwen_reserve_max_users"]["value"]


def test_dense_over_reservation(pages):
    d = pages["dense_waste_fraction"]
    assert cap.dense_waste_fraction(d["mean_len"], d["s_max"]) == d["value"] == 15 / 16
    g = pages["dense_waste_gb"]
    assert math.floor(g["cache_gb"] * d["value"]) == g["value"]


def test_padding_factors(pages):
    p = pages["padding_factors"]
    a, b, c = p["lengths"]
    assert cap.padding_factor(b, a) == p["a_over"]
    assert cap.padding_factor(b, c) == p["c_over"]


def test_internal_fragmentation_bound(pages):
    m = pages["max_tail_waste_rows"]
    bs = m["block_tokens"]
    assert max(cap.tail_waste_slots(n, bs) for n in range(1, 10 * bs)) == m["value"]
    assert cap.tail_waste_slots(0, bs) == 0 and cap.tail_waste_slots(bs, bs) == 0
    assert cap.blocks_for_tokens(17, 16) == 2
