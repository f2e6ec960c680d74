"""Seeded input generators: determinism, shapes and rounding (CPU)."""

import numpy as np

from workloads import config_by_name, draw_normal_storage, storage_from_f32
from workloads.churn import choose_churn, draw_prefix_shared_plan
from workloads.configs import PREFIX_SHARED, draw_decode_shapes


def test_tiny_config_shapes():
    sh = draw_decode_shapes(config_by_name("tiny_f32"))
    assert list(sh.lens) == [5, 17, 33, 60]
    assert sh.num_blocks == 32 and sorted(sh.free_order) == list(range(32))


def test_gpt_lengths_range_and_pool():
    cfg = config_by_name("gpt_f16")
    sh = draw_decode_shapes(cfg)
    assert len(sh.lens) == 64 and sh.lens.min() >= 1 and sh.lens.max() <= 2048
    need = sum(-(-int(L) // 16) for L in sh.lens)
    assert sh.num_blocks == int(np.ceil(1.25 * need))
    assert 250 < sh.lens.mean() < 800


def test_ragged_lengths_include_pinned_values():
    sh = draw_decode_shapes(config_by_name("ragged_bf16"))
    assert len(sh.lens) == 96
    for v in (60, 200, 1500):
        assert v in sh.lens
    assert sh.lens.min() >= 5 and sh.lens.max() <= 10000


def test_gqa_config():
    cfg = config_by_name("gqa_long_bf16")
    sh = draw_decode_shapes(cfg)
    assert list(sh.lens) == [32768] * 10 and cfg.group == 4
    assert cfg.num_kv_heads * cfg.head_dim * 2 * 2 == 4096  # 4 KiB K+V per token


def test_draws_are_deterministic_and_thread_independent():
    a = draw_normal_storage((7, 1), (3, 5, 1 << 20), "bf16", threads=1)
    b = draw_normal_storage((7, 1), (3, 5, 1 << 20), "bf16", threads=8)
    assert a.dtype == np.uint16 and np.array_equal(a, b)


def test_bf16_round_to_nearest_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -1.5], dtype=np.float32)
    got = storage_from_f32(x, "bf16")
    assert list(got) == [0x3F80, 0x3F82, 0x3F81, 0xBFC0]


def test_prefix_shared_plan_and_churn():
    cfg = PREFIX_SHARED
    plan = draw_prefix_shared_plan(cfg)
    assert len(plan.tails) == 256 and plan.tails.min() >= 0 and plan.tails.max() <= 1024
    assert cfg.churn == 13
    live = list(range(1, 257))
    r, p = choose_churn(cfg, 0, live)
    assert len(r) == 13 == len(set(r)) and not set(r) & set(p) and len(set(p)) == 13
    assert choose_churn(cfg, 0, live) == (r, p)
