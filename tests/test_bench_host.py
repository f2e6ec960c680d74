"""Host-side pieces of bench.py (CPU): the one-GPU refusal, the committed
counter summaries it scales its traffic from, and the prefix-shared loop's
churn draws (taken before the timed region) against the seeded choice the
oracle run uses."""

import os
import subprocess
import sys

import numpy as np

import bench
from workloads.churn import apply_churn, choose_churn, draw_churn
from workloads.configs import PREFIX_SHARED

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counter_summary_fields_are_read_only_for_the_matching_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    f = tmp_path / "profiles" / "x_counters.txt"
    f.write_text("# comment: not a field\nkernel_source_sha: abc\nhbm_bytes_per_launch: 1024\n"
                 "algorithmic_bytes_per_launch: 1000\n")
    assert bench.committed_traffic("profiles/x_counters.txt", sha="abc") == 1024.0
    assert abs(bench.committed_traffic_ratio("profiles/x_counters.txt", sha="abc") - 1.024) < 1e-12
    assert bench.committed_traffic("profiles/x_counters.txt", sha="other") is None
    assert bench.committed_traffic_ratio("profiles/x_counters.txt", sha="other") is None
    assert bench.committed_traffic("profiles/missing.txt", sha="abc") is None


def test_churn_draws_taken_ahead_equal_the_seeded_choice():
    cfg = PREFIX_SHARED
    rng = np.random.default_rng(11)
    for it in range(40):
        live = rng.choice(20 * cfg.num_seqs, size=cfg.num_seqs, replace=False)
        want = choose_churn(cfg, it, live.tolist())
        got = apply_churn(live.astype(np.int32), *draw_churn(cfg, it, cfg.num_seqs))
        assert got == want
        retire, parents = got
        assert len(set(retire)) == cfg.churn and not set(retire) & set(parents)
