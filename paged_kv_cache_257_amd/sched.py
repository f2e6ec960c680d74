"""Python binding of the continuous-batching scheduler (pkv_sched_*), plus a
command-line run that reports the pool and request metrics the lesson lists
(free/used blocks, allocation failures, tail waste, prefix hit rate,
preemptions, queue delay, time to first token and inter-token latency, per
request class) and the scheduler's host time per iteration.

    python -m paged_kv_cache_257_amd.sched [--requests N] [--blocks B] [--json]
"""

from __future__ import annotations

import argparse
import ctypes as C
import json
import sys
import time
from typing import List

import numpy as np

from ._capi import (Request, RequestState, SchedConfig, SchedItem, SchedStats, SchedStepInfo,
                    check)
from .pool import Pool


class Scheduler:
    def __init__(self, pool: Pool, requests: List[dict], max_batch_tokens: int, chunk_tokens: int,
                 max_running: int):
        self.pool = pool
        self.lib = pool.lib
        self.n = len(requests)
        arr = (Request * max(self.n, 1))()
        for i, r in enumerate(requests):
            arr[i] = Request(r["arrival"], r["prompt_len"], r["output_len"], r.get("klass", 0),
                             r.get("prefix_id", -1), r.get("prefix_len", 0))
        self.cfg = SchedConfig(max_batch_tokens, chunk_tokens, max_running)
        self.items = (SchedItem * max_running)()
        self.cap = max_running
        self._info = SchedStepInfo()
        h = C.c_void_p()
        check(self.lib, self.lib.pkv_sched_create(pool.handle, C.byref(self.cfg), arr, self.n, C.byref(h)))
        self.handle = h

    def close(self) -> None:
        if getattr(self, "handle", None):
            self.lib.pkv_sched_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 -- interpreter shutdown
            pass

    def step(self):
        """One iteration: (items [(request, seq, kind, pos, n)], events dict)."""
        check(self.lib, self.lib.pkv_sched_step(self.handle, self.items, self.cap, C.byref(self._info)))
        k = self._info.n_items
        items = [(it.request, it.seq, it.kind, it.pos, it.n_tokens) for it in self.items[:k]]
        return items, self._info.as_dict()

    def step_raw(self) -> int:
        """One iteration without converting the items (timing); returns the item count."""
        check(self.lib, self.lib.pkv_sched_step(self.handle, self.items, self.cap, C.byref(self._info)))
        return self._info.n_items

    def request(self, i: int) -> dict:
        s = RequestState()
        check(self.lib, self.lib.pkv_sched_request(self.handle, i, C.byref(s)))
        return s.as_dict()

    def stats(self) -> dict:
        s = SchedStats()
        check(self.lib, self.lib.pkv_sched_stats(self.handle, C.byref(s)))
        return s.as_dict()

    def done(self) -> bool:
        st = self.stats()
        return st["finished"] + st["rejected"] == self.n


def request_metrics(requests: List[dict], states: List[dict]) -> dict:
    """Per-class queue delay, time to first token and inter-token latency
    (iterations) of finished requests."""
    out = {}
    for k in sorted({r.get("klass", 0) for r in requests}):
        rows = [(r, s) for r, s in zip(requests, states) if r.get("klass", 0) == k and s["finished_at"] >= 0]
        if not rows:
            continue
        qd = np.array([s["admitted_at"] - r["arrival"] for r, s in rows], dtype=float)
        ttft = np.array([s["first_token_at"] - r["arrival"] for r, s in rows], dtype=float)
        itl = np.array([(s["finished_at"] - s["first_token_at"]) / (r["output_len"] - 1)
                        for r, s in rows if r["output_len"] > 1], dtype=float)
        out[k] = {"finished": len(rows), "queue_delay_mean": round(float(qd.mean()), 2),
                  "ttft_mean": round(float(ttft.mean()), 2), "ttft_p90": round(float(np.percentile(ttft, 90)), 2),
                  "itl_mean": round(float(itl.mean()), 3) if len(itl) else None,
                  "preempted_requests": sum(1 for _, s in rows if s["preemptions"] > 0)}
    return out


def main(argv=None) -> int:
    from workloads.requests import draw_request_trace
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--requests", type=int, default=2000)
    ap.add_argument("--blocks", type=int, default=6000, help="K/V pool blocks of 16 tokens")
    ap.add_argument("--max-batch-tokens", type=int, default=4096)
    ap.add_argument("--chunk", type=int, default=512)
    ap.add_argument("--max-running", type=int, default=256)
    ap.add_argument("--rate", type=float, default=0.15, help="arrivals per iteration (6000 blocks serve ~0.19)")
    ap.add_argument("--seed", type=int, default=42)
    ap.add_argument("--json", action="store_true")
    a = ap.parse_args(argv)
    reqs = draw_request_trace(a.requests, a.seed, rate=a.rate)
    width = -(-(4096 + 2048) // 16)
    pool = Pool(a.blocks, 1, 8, "f16", width, 16, host_only=True)
    sch = Scheduler(pool, reqs, a.max_batch_tokens, a.chunk, a.max_running)
    host_s, steps, peak_used = 0.0, 0, 0
    waste, fails = [], 0
    while not sch.done():
        t = time.perf_counter()
        sch.step_raw()
        host_s += time.perf_counter() - t
        steps += 1
        ps = pool.stats()
        peak_used = max(peak_used, ps["used_blocks"])
        waste.append(ps["tail_waste_slots"])
    sch.step_raw()  # the last finished sequences leave at the next iteration boundary
    st = sch.stats()
    states = [sch.request(i) for i in range(len(reqs))]
    ps = pool.stats()
    res = {"iterations": steps, "host_us_per_iteration": round(host_s / max(steps, 1) * 1e6, 2),
           "finished": st["finished"], "rejected": st["rejected"], "preemptions": st["preemptions"],
           "prefix_hit_rate": round(st["prefix_hit_tokens"] / max(st["prompt_tokens_admitted"], 1), 4),
           "prefill_tokens": st["prefill_tokens"], "decode_tokens": st["decode_tokens"],
           "pool": {"blocks": a.blocks, "peak_used_blocks": peak_used, "free_blocks_end": ps["free_blocks"],
                    "alloc_failures": ps["alloc_failures"],
                    "mean_tail_waste_slots": round(float(np.mean(waste)), 1) if waste else 0.0},
           "per_class": request_metrics(reqs, states)}
    sch.close()
    pool.close()
    print(json.dumps(res) if a.json else json.dumps(res, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
