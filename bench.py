"""Benchmark: paged decode on one MI355X, GPT-style 64-sequence fp16 batch.

A step is one decode iteration of the whole path over one batch:
  host   pkv_prepare_decode (C++): append one token to each of the 64
         sequences, take copy-on-write pairs, build block tables, lengths and
         the split-K plan into a pinned staging buffer; one async upload;
  device copy_blocks (if any pairs), then one paged-decode launch that stores
         the 64 new tokens' K/V and attends (split-K partials combined in the
         same launch); the step's metadata uploads on a side stream while the
         previous step computes.  The whole step is one native call
         (pkv_stepper_step); --two-launch / --separate-write / --no-overlap
         switch fusions off for comparison.
Inputs (pools, q, the new tokens' K/V) are resident in HBM before timing.
``--replicas`` independent copies of the batch (own pools, own allocators)
are stepped in rotation so that every step reads K/V that the previous
steps have pushed out of L2 and the 256 MiB Infinity Cache.

Reported (one JSON line):
  value        K/V bytes the steps attended / wall time of the K steps (GB/s);
  roofline     the decode launches of the K timed steps: algorithmic K/V
               bytes per launch / average launch duration, the span of the
               decode stream between two HIP events around the timed steps
               divided by K (so each dispatch's idle gap counts as
               duration), against the 8 TB/s HBM peak; after the timed
               steps, as many more launches (at least 20) each carry their
               own events for the spread of single-kernel durations;
               ``traffic`` scales the committed rocprofv3 counter summary's
               ratio (FETCH_SIZE + WRITE_SIZE over algorithmic bytes) by this
               line's bytes, while the kernel source is the profiled one;
  cpu_baseline the fp64 CPU oracle on a bounded sample of the same batch.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from typing import Optional

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "paged-decode achieved HBM GB/s (% of peak) + decode tokens/s, 64-seq fp16 batch"
# the headline metric names the GPT-style 64-sequence fp16 batch; every other
# decode workload reports the same quantities under its own description
DECODE_METRICS = {
    "gpt_f16": METRIC,
    "tiny_f32": "paged-decode achieved HBM GB/s (% of peak) + decode tokens/s, tiny 4-seq fp32 batch",
    "ragged_bf16": "paged-decode achieved HBM GB/s (% of peak) + decode tokens/s, 96-seq ragged bf16 batch",
    "gqa_long_bf16": "paged-decode achieved HBM GB/s (% of peak) + decode tokens/s, "
                     "10 x 32768-token GQA-4 bf16 batch",
}
PREFIX_METRIC = ("prefix-shared decode loop: logical K/V GB/s + iteration tokens/s, "
                 "256 seqs over one 4096-token prefix, fp16")
KERNEL_SOURCES = ("paged_kv_cache_257_amd/csrc/kernels/paged_decode.hip",
                  "paged_kv_cache_257_amd/csrc/kernels/device_common.h",
                  "paged_kv_cache_257_amd/csrc/kernels/mfma_common.h")
COUNTER_SUMMARY = "profiles/paged_decode_gpt_f16_counters.txt"


def counter_summary(workload: str) -> str:
    """The committed HBM-counter summary of a decode workload."""
    return f"profiles/paged_decode_{workload}_counters.txt"


def decode_kernel_name(dtype: str, head_dim: int, group: int) -> str:
    """The kernel that runs a decode launch: grouped-query fp16/bf16 batches
    of head_dim 128 go to the matrix-core kernel unless PKV_DECODE_MFMA=0."""
    if group >= 2 and head_dim == 128 and dtype in ("f16", "bf16") and \
            os.environ.get("PKV_DECODE_MFMA", "1")[:1] != "0":
        return "paged_decode_mfma_kernel"
    return "paged_decode_kernel"


def kernel_source_sha() -> str:
    return _sources_sha(KERNEL_SOURCES)


PREFILL_SOURCES = ("paged_kv_cache_257_amd/csrc/kernels/paged_prefill.hip",
                   "paged_kv_cache_257_amd/csrc/kernels/device_common.h",
                   "paged_kv_cache_257_amd/csrc/kernels/mfma_common.h")


def _sources_sha(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def prefill_source_sha() -> str:
    return _sources_sha(PREFILL_SOURCES)


def _summary_fields(summary: str, sha: Optional[str]):
    path = os.path.join(ROOT, summary)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != (sha or kernel_source_sha()):
        return None
    return kv


def committed_traffic(summary: str = COUNTER_SUMMARY, sha: Optional[str] = None,
                      key: str = "hbm_bytes_per_launch"):
    """HBM bytes from a committed counter summary, if it was taken on the
    current kernel source (else None)."""
    kv = _summary_fields(summary, sha)
    try:
        return float(kv[key]) if kv else None
    except (KeyError, ValueError):
        return None


def committed_traffic_ratio(summary: str, sha: Optional[str] = None):
    """Counter bytes per algorithmic byte of the profiled run (HBM traffic
    FETCH + WRITE, calibrated, over the K/V bytes the same launches attended),
    if the summary was taken on the current kernel source.  A line scales it
    by its own algorithmic bytes: the profiled run's contexts may have grown
    further than this line's."""
    kv = _summary_fields(summary, sha)
    if not kv:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"]) / float(kv["algorithmic_bytes_per_launch"])
    except (KeyError, ValueError, ZeroDivisionError):
        return None


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="gpt_f16")
    ap.add_argument("--partition", type=int, default=-1,
                    help="split-K partition tokens (0 = library default; -1 = fill mode: per step, the "
                         "smallest partition whose workgroups are all resident at once, else the default)")
    ap.add_argument("--max-keys", type=int, default=None,
                    help="prefill workloads: split tiles attending more keys (0 = never, -1 = the "
                         "library's rule for under-filled launches; default -1)")
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--two-launch", action="store_true",
                    help="decode as partition kernel + separate combine kernel (comparison)")
    ap.add_argument("--separate-write", action="store_true",
                    help="store the new tokens with write_kv instead of inside the decode (comparison)")
    ap.add_argument("--no-overlap", action="store_true",
                    help="upload each step's metadata on the compute stream (comparison)")
    ap.add_argument("--time-every", type=int, default=1,
                    help="prefix-shared loop: attach HIP timing events to every N-th iteration's decode")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--gather-probe", action="store_true",
                    help="time the decode launch of the workload's batch beside the gather probe "
                         "(the same tile reads without the arithmetic) in each staging mode, and the "
                         "register-staged decode instance where the default stages through LDS; "
                         "prints one JSON line")
    return ap.parse_args(argv)


def calib_copy():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": n, "launches": 3}))


def bench_gather_probe(args, cfg):
    """The decode launch of the workload's batch (contexts as drawn, no
    append) against the gather probe on the same tables and plan: the rate
    of the decode's own tile reads with no arithmetic, per staging mode.
    Each kernel runs N times back to back between two events on the launch
    stream; its time is the span / N."""
    import numpy as np
    import torch

    from paged_kv_cache_257_amd import Pool, decode_plan, decode_workspace_bytes
    from paged_kv_cache_257_amd.pool import fill_partition
    from workloads import draw_decode_values
    from workloads.configs import draw_decode_shapes

    sh = draw_decode_shapes(cfg)
    vals = draw_decode_values(cfg, sh.lens)
    B, Hq, H, d, dt = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.dtype
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]

    def dev(bits):
        a = np.ascontiguousarray(bits)
        t = torch.from_numpy(a.view(np.int16) if dt == "bf16" else a)
        return (t.view(torch.bfloat16) if dt == "bf16" else t).to("cuda")

    stride = -(-int(sh.lens.max()) // 16)
    kc = torch.zeros((sh.num_blocks, H, 16, d), dtype=tdt, device="cuda")
    vc = torch.zeros_like(kc)
    pool = Pool(sh.num_blocks, H, d, dt, stride, 16, sh.free_order, kc, vc)
    slots = np.concatenate([pool.alloc(int(L))[1] for L in sh.lens])
    pool.write_kv(dev(vals["k"]), dev(vals["v"]), torch.from_numpy(slots).cuda())
    tables, lens = pool.build_batch(list(range(B)), stride)
    if args.partition == -1:
        P = fill_partition(lens, *pool.decode_occupancy(Hq)) or 0
    else:
        P = args.partition
    plan, info = decode_plan(lens, P)
    t_d, l_d, p_d = (torch.from_numpy(a).cuda() for a in (tables, lens, plan))
    q = dev(vals["q"])
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(decode_workspace_bytes(info, Hq, d) // 4, 1), dtype=torch.float32, device="cuda")
    probe_out = torch.empty(info.n_work * H * 4, dtype=torch.int32, device="cuda")
    per_tok = 2 * H * d * cfg.elem_bytes
    alg = int(lens.sum()) * per_tok
    tile_bytes = int(sum(-(-int(L) // 16) for L in lens)) * 16 * per_tok
    n = max(args.steps, 50)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(max(args.warmup, 5)):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        return {"us": round(ms * 1e3, 2), "GBps": round(alg / ms / 1e6, 1),
                "frac": round(alg / ms / 1e6 / HBM_PEAK_GBPS, 4)}

    def decode():
        pool.paged_decode(q, out, t_d, l_d, cfg.scale, p_d, info, ws)

    res = {"mode": "gather_probe", "workload": cfg.name, "dtype": dt, "launches": n,
           "partition_tokens": info.partition_tokens, "work_items": info.n_work,
           "algorithmic_bytes": alg, "tile_bytes": tile_bytes, "kernels": {}}
    res["kernels"]["decode"] = timed(decode)
    tile = 16 * d * cfg.elem_bytes
    if Hq == H and d == 128 and dt in ("f16", "bf16"):
        # the default instance stages tiles through LDS; the register-staged
        # one beside it
        os.environ["PKV_DECODE_STAGING"] = "regs"
        try:
            res["kernels"]["decode_regs_staged"] = timed(decode)
        finally:
            del os.environ["PKV_DECODE_STAGING"]
    # the probe in each staging mode at 4 and 2 waves per workgroup; the
    # register modes also with 64 KiB of unused LDS per workgroup, which
    # caps a CU at two workgroups as the LDS stages do (the register probe
    # needs few registers and otherwise runs many more per CU)
    for mode in ("regs", "cached", "lds"):
        if mode == "lds" and tile > 4096:
            continue
        for waves in (4, 2):
            for pad in ((0,) if mode == "lds" else (0, 65536)):
                key = f"probe_{mode}_w{waves}" + ("_pad64k" if pad else "")
                res["kernels"][key] = timed(
                    lambda: pool.gather_probe(t_d, l_d, p_d, info, probe_out, mode, waves, pad))
    best = max(v["GBps"] for k, v in res["kernels"].items() if k.startswith("probe_"))
    res["gather_ceiling_GBps"] = best
    res["decode_frac_of_ceiling"] = round(res["kernels"]["decode"]["GBps"] / best, 4)
    print(json.dumps(res))
    pool.close()
    return 0


def cpu_baseline(cfg, sh, vals, stride, budget_s):
    """The fp64 oracle on a bounded sample of the same batch."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle.runs import DecodeRun

    cores = os.cpu_count() or 1
    with threadpool_limits(limits=cores):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        run = DecodeRun(cfg, sh.lens, sh.num_blocks, sh.free_order, stride)
        run.write_context(vals["k"], vals["v"])
        order = np.random.default_rng(cfg.seed + 7).permutation(len(sh.lens))
        # whole passes over the batch in a fixed random order until the
        # budget is spent (the last pass may be partial)
        done, tokens, t0 = 0, 0, time.perf_counter()
        while time.perf_counter() - t0 <= budget_s:
            i = int(order[done % len(order)])
            run.attend(i, vals["q"][i])
            done += 1
            tokens += int(sh.lens[i])
        dt = time.perf_counter() - t0
    kv_bytes = tokens * 2 * cfg.num_kv_heads * cfg.head_dim * cfg.elem_bytes
    return {"value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{done / len(sh.lens):.2f} passes over the {len(sh.lens)}-sequence batch "
                      f"({done} sequence decodes, {tokens} context tokens), fp64 numpy attention, "
                      f"{dt:.1f} s",
            "decode_tokens_per_s": round(done / dt, 3)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_probe():
    """A plain 1 GiB device-to-device copy timed with HIP events: the GB/s
    (read + write) a streaming kernel reaches on this GPU, for context."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms = []
    for _ in range(5):
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    del src, dst
    torch.cuda.empty_cache()
    best = min(ms)
    return {"bytes_moved": 2 * n, "ms_best": round(best, 4), "GBps": round(2 * n / best / 1e6, 1)}


def event_launches(args) -> int:
    """Decode launches timed one by one after the K timed steps: K, at
    least 20 and at most 400."""
    return max(20, min(args.steps, 400))


def timing_events(n: int):
    """n (start, stop) timing-event pairs whose HIP events already exist.
    torch creates a HIP event at its first record; recording each pair once
    here keeps those creations and their extra stream markers out of the
    timed region (the stepper attaches the pair to a dispatch itself)."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record()
        b.record()
    torch.cuda.synchronize()
    return ev


def prefix_shared_schedule(cfg, plan, width, iterations):
    """Replay the prefix-shared loop on a host-only allocator (the same C++
    allocator, no GPU) to count each iteration's bytes: logical = every
    decoded sequence's context, physical = the distinct filled slots those
    contexts map to (shared prefix blocks counted once)."""
    import numpy as np

    from paged_kv_cache_257_amd import Pool
    from workloads.churn import choose_churn

    pool = Pool(plan.num_blocks, cfg.num_kv_heads, cfg.head_dim, cfg.dtype, width, 16,
                plan.free_order, host_only=True)
    try:
        root, _ = pool.alloc(cfg.prefix_len)
        for t in plan.tails:
            pool.append(pool.fork(root), int(t))
        rows, col = [], np.arange(width)
        for it in range(iterations):
            seqs = [x for x in pool.live() if x != root]
            pool.append_batch(seqs, 1)
            pool.take_cow()
            tables, lens = pool.build_batch(seqs, width)
            fill = np.clip(lens[:, None] - 16 * col[None, :], 0, 16)
            used = fill > 0
            blocks, fills = tables[used], fill[used]
            best = np.zeros(plan.num_blocks, dtype=np.int64)
            np.maximum.at(best, blocks, fills)
            rows.append((len(seqs), int(lens.sum()), int(best.sum())))
            retire, parents = choose_churn(cfg, it, seqs)
            for x in retire:
                pool.free(x)
            for x in parents:
                pool.fork(x)
        return rows
    finally:
        pool.close()


def bench_prefix_shared(args, cfg):
    """The prefix-shared continuous-batching loop: every iteration appends one
    token to each of the 256 decoding sequences (copy-on-write where a
    partly filled block is shared), decodes them all, retires 13 and admits
    13 forks.  The timed region is whole iterations, CPU scheduler work
    included."""
    import numpy as np
    import torch

    from paged_kv_cache_257_amd import Pool
    from paged_kv_cache_257_amd.step import DecodeIteration
    from workloads import draw_normal_storage
    from workloads.churn import apply_churn, draw_churn, draw_prefix_shared_plan

    warm = min(args.warmup, 8)
    steps = min(args.steps, cfg.iterations - warm)
    total = warm + steps
    plan = draw_prefix_shared_plan(cfg)
    width = -(-(cfg.prefix_len + cfg.tail_max + cfg.iterations) // 16)
    H, Hq, d, dt = cfg.num_kv_heads, cfg.num_q_heads, cfg.head_dim, cfg.dtype
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]
    per_tok = 2 * H * d * (4 if dt == "f32" else 2)
    sched = prefix_shared_schedule(cfg, plan, width, total)

    def dev(bits):
        a = np.ascontiguousarray(bits)
        t = torch.from_numpy(a.view(np.int16) if dt == "bf16" else a)
        return (t.view(torch.bfloat16) if dt == "bf16" else t).to("cuda")

    kc = torch.zeros((plan.num_blocks, H, 16, d), dtype=tdt, device="cuda")
    vc = torch.zeros_like(kc)
    pool = Pool(plan.num_blocks, H, d, dt, width, 16, plan.free_order, kc, vc)
    # context K/V: a seeded 8192-token chunk written over and over (values do
    # not change the traffic)
    chunk = 8192
    ck = dev(draw_normal_storage((cfg.seed, 60), (chunk, H, d), dt))
    cv = dev(draw_normal_storage((cfg.seed, 61), (chunk, H, d), dt))
    root, slots = pool.alloc(cfg.prefix_len)
    all_slots = [slots] + [pool.append(pool.fork(root), int(t)) for t in plan.tails]
    all_slots = torch.from_numpy(np.concatenate(all_slots)).cuda()
    for o in range(0, all_slots.numel(), chunk):
        sl = all_slots[o:o + chunk]
        pool.write_kv(ck[:sl.numel()], cv[:sl.numel()], sl)
    del ck, cv
    n_max = cfg.num_seqs
    vals = [(dev(draw_normal_storage((cfg.seed, 70 + j), (n_max, Hq, d), dt)),
             dev(draw_normal_storage((cfg.seed, 80 + j), (n_max, H, d), dt)),
             dev(draw_normal_storage((cfg.seed, 90 + j), (n_max, H, d), dt))) for j in range(4)]
    out = torch.empty((n_max, Hq, d), dtype=torch.float32, device="cuda")
    step = DecodeIteration(pool, n_max, width, Hq, args.partition)
    ev = timing_events(total)
    torch.cuda.synchronize()

    # the seeded retire / fork draws are workload input, drawn before the
    # loop like the K/V values (every iteration decodes num_seqs sequences)
    draws = [draw_churn(cfg, it, cfg.num_seqs) for it in range(total)]

    def iteration(it):
        live = np.asarray(pool.live(), dtype=np.int32)
        seqs = live[live != root]
        assert len(seqs) == cfg.num_seqs
        q, k, v = vals[it % 4]
        lay = step.step(seqs, q, out, k, v, cfg.scale, events=ev[it] if it % every == 0 else None)
        loads.append(lay.plan.shared_kv)
        retire, parents = apply_churn(seqs, *draws[it])
        pool.free_batch(retire)
        pool.fork_batch(parents)
        return len(seqs)

    loads = []  # the plan's load-policy hint of every iteration
    # an iteration is ~1 ms, so timing events on every decode cost little
    every = max(1, args.time_every)
    for it in range(warm):
        iteration(it)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    decoded = sum(iteration(it) for it in range(warm, total))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stats = pool.stats()
    step.close()
    pool.close()
    timed = range(warm, total)
    assert decoded == sum(sched[i][0] for i in timed)
    logical = sum(sched[i][1] for i in timed) * per_tok
    physical = sum(sched[i][2] for i in timed) * per_tok
    sampled = [i for i in timed if i % every == 0]
    kern_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in sampled]
    s_log = float(np.mean([sched[i][1] for i in sampled])) * per_tok
    s_phy = float(np.mean([sched[i][2] for i in sampled])) * per_tok
    km = float(np.mean(kern_ms)) / 1e3 if kern_ms else float("nan")
    ratio = committed_traffic_ratio(counter_summary(cfg.name)) if args.partition == -1 else None
    res = {
        "metric": PREFIX_METRIC,
        "value": round(logical / wall / 1e9, 2),
        "unit": "GB/s (logical)",
        "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(wall / steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic",
        "config": {"workload": cfg.name, "num_seqs": cfg.num_seqs, "num_q_heads": Hq, "num_kv_heads": H,
                   "head_dim": d, "block_size": 16, "prefix_len": cfg.prefix_len,
                   "tail_max": cfg.tail_max, "churn_per_iteration": cfg.churn,
                   "step": "append + copy-on-write + decode (new K/V stored inside) + retire/admit",
                   "kv_loads": "cached" if all(loads[warm:]) else
                   "streaming" if not any(loads[warm:]) else "mixed"},
        "physical_GBps": round(physical / wall / 1e9, 2),
        "pct_of_hbm_peak_physical": round(100 * physical / wall / 1e9 / HBM_PEAK_GBPS, 2),
        "iteration_tokens_per_s": round(decoded / wall, 1),
        "cow_copies": stats["cow_copies"],
        # the decode of an iteration (every launch it makes), timed with HIP
        # events on its stream; bytes are the distinct K/V the decoded
        # contexts map to (a block shared by many sequences counted once):
        # what one pass must read from HBM at the least
        "roofline": {"bound": "hbm", "achieved": round(s_phy / km / 1e9, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(s_phy / km / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": round(ratio * s_phy) if ratio else None,
                     "traffic_ratio": round(ratio, 4) if ratio else None,
                     "bytes": "distinct K/V per iteration",
                     "kernel_ms_mean": round(km * 1e3, 4),
                     "kernel_ms_median": round(float(np.median(kern_ms)), 4),
                     "kernel_ms_p10": round(float(np.percentile(kern_ms, 10)), 4),
                     "kernel_ms_p90": round(float(np.percentile(kern_ms, 90)), 4),
                     "timed_launches": len(kern_ms), "time_every": every,
                     "algorithmic_bytes_per_launch": int(s_phy),
                     "logical_bytes_per_launch": int(s_log),
                     "logical_GBps": round(s_log / km / 1e9, 1),
                     "kernel_source_sha": kernel_source_sha()},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = prefix_cpu_baseline(cfg, plan, width, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


def prefix_cpu_baseline(cfg, plan, width, budget_s):
    """The fp64 oracle on a bounded sample of the prefix-shared loop: the
    oracle allocator and mirrored pool are set up as the loop starts and
    the first iteration's append is replayed (not timed); then seeded
    decoding sequences attend with that iteration's queries until the
    budget is spent.  Rate in the line's unit: logical K/V bytes attended
    per second."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle.runs import PrefixSharedRun, iteration_values, prefix_values

    cores = os.cpu_count() or 1
    with threadpool_limits(limits=cores):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        ora = PrefixSharedRun(cfg, plan, width, with_mirror=True)
        ora.setup(prefix_values(cfg, plan.tails))
        seqs, slots, cow = ora.append_step()
        q, k, v = iteration_values(cfg, 0, len(seqs))
        ora.write_step(cow, k, v, slots)
        order = np.random.default_rng(cfg.seed + 7).permutation(len(seqs))
        done, tokens, t0 = 0, 0, time.perf_counter()
        while time.perf_counter() - t0 <= budget_s:
            i = int(order[done % len(order)])
            ora.attend(seqs[i], q[i])
            done += 1
            tokens += ora.alloc.length(seqs[i])
        dt = time.perf_counter() - t0
    per_tok = 2 * cfg.num_kv_heads * cfg.head_dim * (4 if cfg.dtype == "f32" else 2)
    return {"value": round(tokens * per_tok / dt / 1e9, 4), "unit": "GB/s (logical)", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{done} sequence decodes of the loop's first iteration ({tokens} context tokens), "
                      f"fp64 numpy attention through the oracle allocator, {dt:.1f} s",
            "decode_tokens_per_s": round(done / dt, 3)}


MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 matrix-core peak
PREFILL_MAX_KEYS = -1      # prefill key split: -1 = the library's rule (only under-filled launches)


def prefill_flops(q_len: int, ctx_len: int, num_q_heads: int, head_dim: int) -> int:
    """Algorithmic flops of causal attention for one chunk: every (query,
    visible key) pair costs 2 d for q.k and 2 d for p.v, per query head."""
    C = ctx_len - q_len
    pairs = q_len * C + q_len * (q_len + 1) // 2
    return 4 * head_dim * num_q_heads * pairs


def bench_prefill(args, cfg):
    """Chunked prefill of a workload's prompts.  All chunks' K/V are written
    first (blocks never move once allocated, so step k's tables are the
    prefix of the final ones); a bench step is then the whole chunk
    schedule, one prefill launch per chunk step with that step's context
    lengths.  Two rooflines: the matrix cores (causal attention's flops at
    the dense fp16/bf16 peak) and HBM (each launch reads at least the K/V of
    every key its chunks attend, the whole context up to each chunk's end,
    once, and writes its fp32 output); the line reports the one whose time
    is larger, the other beside it."""
    import numpy as np
    import torch

    from paged_kv_cache_257_amd import Pool, prefill_plan, prefill_workspace_bytes
    from workloads import draw_normal_storage
    from workloads.prefill import draw_prefill_shapes

    max_keys = PREFILL_MAX_KEYS if args.max_keys is None else args.max_keys

    sh = draw_prefill_shapes(cfg)
    H, Hq, d, dt = cfg.num_kv_heads, cfg.num_q_heads, cfg.head_dim, cfg.dtype
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dt]
    width = -(-int(sh.prompts.max()) // 16)

    def dev(bits):
        a = np.ascontiguousarray(bits)
        t = torch.from_numpy(a.view(np.int16) if dt == "bf16" else a)
        return (t.view(torch.bfloat16) if dt == "bf16" else t).to("cuda")

    kc = torch.zeros((sh.num_blocks, H, 16, d), dtype=tdt, device="cuda")
    vc = torch.zeros_like(kc)
    pool = Pool(sh.num_blocks, H, d, dt, width, 16, sh.free_order, kc, vc)
    slots = []
    for step in sh.steps:
        for seq, t0, n in step:
            if t0 == 0:
                sid, s_ = pool.alloc(n)
                assert sid == seq
            else:
                s_ = pool.append(seq, n)
            slots.append(s_)
    slots = torch.from_numpy(np.concatenate(slots)).cuda()
    # K/V: a seeded 8192-token chunk written over and over (values do not
    # change the work)
    chunk = 8192
    ck = dev(draw_normal_storage((cfg.seed, 60), (chunk, H, d), dt))
    cv = dev(draw_normal_storage((cfg.seed, 61), (chunk, H, d), dt))
    for o in range(0, slots.numel(), chunk):
        sl = slots[o:o + chunk]
        pool.write_kv(ck[:sl.numel()], cv[:sl.numel()], sl)
    del ck, cv
    launches, flops, kv_bytes, ws_bytes = [], [], [], 0
    per_tok = 2 * H * d * cfg.elem_bytes
    max_q = max(sum(n for _, _, n in step) for step in sh.steps)
    q_all = dev(draw_normal_storage((cfg.seed, 62), (max_q, Hq, d), dt))
    out = torch.empty((max_q, Hq, d), dtype=torch.float32, device="cuda")
    for step in sh.steps:
        seqs = [x for x, _, _ in step]
        q_lens = np.array([n for _, _, n in step])
        lens = np.array([t0 + n for _, t0, n in step], dtype=np.int32)
        tables, _ = pool.build_batch(seqs, width)
        plan, info = prefill_plan(q_lens, lens, Hq, H, max_keys)
        launches.append((torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(),
                         torch.from_numpy(plan).cuda(), info, int(q_lens.sum())))
        ws_bytes = max(ws_bytes, prefill_workspace_bytes(info, d))
        flops.append(sum(prefill_flops(int(n), int(L), Hq, d) for n, L in zip(q_lens, lens)))
        # K/V of every attended key once, q read, fp32 out written
        kv_bytes.append(int(lens.sum()) * per_tok + int(q_lens.sum()) * Hq * d * (cfg.elem_bytes + 4))
    total_tokens = int(sh.prompts.sum())
    # zeroed once: every launch leaves the split tiles' tickets at zero
    workspace = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in launches] for _ in range(args.warmup + args.steps)]

    def schedule(r):
        for k, (tb, ln, pl, info, nq) in enumerate(launches):
            ev[r][k][0].record()
            pool.paged_prefill(q_all[:nq], out[:nq], tb, ln, cfg.scale, pl, info, workspace)
            ev[r][k][1].record()

    for r in range(args.warmup):
        schedule(r)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(args.warmup, args.warmup + args.steps):
        schedule(r)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = np.array([[ev[r][k][0].elapsed_time(ev[r][k][1]) for k in range(len(launches))]
                        for r in range(args.warmup, args.warmup + args.steps)])
    per_launch_ms = kern_ms.mean(axis=0)
    total_flops = float(sum(flops))
    total_bytes = float(sum(kv_bytes))
    kern_total_s = float(per_launch_ms.sum()) / 1e3
    t_mfma = total_flops / (MFMA_PEAK_TFLOPS * 1e12)
    t_hbm = total_bytes / (HBM_PEAK_GBPS * 1e9)
    mfma_line = {"bound": "mfma", "achieved": round(total_flops / kern_total_s / 1e12, 2),
                 "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(total_flops / kern_total_s / 1e12 / MFMA_PEAK_TFLOPS, 4),
                 "bound_ms": round(t_mfma * 1e3, 4)}
    hbm_line = {"bound": "hbm", "achieved": round(total_bytes / kern_total_s / 1e9, 2),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(total_bytes / kern_total_s / 1e9 / HBM_PEAK_GBPS, 4),
                "bound_ms": round(t_hbm * 1e3, 4), "algorithmic_bytes_per_step": int(total_bytes)}
    main, other = (hbm_line, mfma_line) if t_hbm > t_mfma else (mfma_line, hbm_line)
    k_big = int(np.argmax(flops))
    pool.close()
    res = {
        "metric": "chunked paged prefill: causal attention TFLOP/s",
        "value": round(total_flops * args.steps / wall / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic",
        "config": {"workload": cfg.name, "prompts": len(sh.prompts), "prompt_tokens": total_tokens,
                   "chunk_tokens": cfg.chunk_tokens, "launches_per_step": len(launches),
                   "max_keys_per_item": max_keys,
                   "split_tiles_per_step": int(sum(l[3].n_split for l in launches)),
                   "num_q_heads": Hq, "num_kv_heads": H, "head_dim": d, "block_size": 16,
                   "accumulate": "f32", "output": "f32"},
        "prompt_tokens_per_s": round(total_tokens * args.steps / wall, 1),
        "roofline": {**main,
                     "other_roofline": other,
                     "traffic": committed_traffic(f"profiles/paged_prefill_{cfg.name}_counters.txt",
                                                  prefill_source_sha(), "hbm_bytes_per_step")
                     if max_keys == PREFILL_MAX_KEYS else None,
                     "traffic_unit": "HBM bytes per step", "kernel": "paged_prefill_kernel",
                     "kernel_ms_per_step": round(float(per_launch_ms.sum()), 4),
                     "largest_launch": {"flops": flops[k_big], "ms": round(float(per_launch_ms[k_big]), 4),
                                        "TFLOPs": round(flops[k_big] / per_launch_ms[k_big] / 1e9, 1)},
                     "algorithmic_flops_per_step": int(total_flops)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = prefill_cpu_baseline(cfg, sh, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


def prefill_cpu_baseline(cfg, sh, budget_s):
    """The fp64 oracle's chunked prefill on a bounded sample of the same
    schedule: each pass replays every chunk step through the oracle
    allocator and mirrored pool (not timed) and attends k seeded query rows
    of each chunk (timed); passes repeat with k doubled until the budget is
    spent."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle.runs import PrefillRun
    from workloads.prefill import draw_prefill_values

    cores = os.cpu_count() or 1
    with threadpool_limits(limits=cores):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        vals = draw_prefill_values(cfg, sh.prompts)
        rng = np.random.default_rng(cfg.seed + 9)
        done, flops, spent, k, passes = 0, 0, 0.0, 4, 0
        while spent <= budget_s:
            run = PrefillRun(cfg, sh, -(-int(sh.prompts.max()) // 16), vals)
            passes += 1
            for _ in sh.steps:
                items = run.append_step()
                for seq, t0, n, _slots in items:
                    rows = sorted(set(rng.integers(0, n, size=min(k, n)).tolist()))
                    t = time.perf_counter()
                    run.attend(seq, t0, n, rows=rows)
                    spent += time.perf_counter() - t
                    done += len(rows)
                    flops += sum(4 * cfg.head_dim * cfg.num_q_heads * (t0 + r + 1) for r in rows)
                if spent > budget_s:
                    break
            k *= 2
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{done} query rows of the same schedule ({passes} passes, seeded rows of "
                      f"every chunk), fp64 numpy causal attention through the oracle allocator, "
                      f"{spent:.1f} s"}


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path runs on one GPU; it is not sharded across GPUs)", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    if args.calib_copy:
        calib_copy()
        return 0

    from paged_kv_cache_257_amd import Pool
    from paged_kv_cache_257_amd.step import DecodeIteration
    from workloads import config_by_name, draw_decode_values, draw_normal_storage
    from workloads.configs import PrefixSharedConfig, draw_decode_shapes

    from workloads.prefill import PREFILL_CONFIGS
    pf = {c.name: c for c in PREFILL_CONFIGS}
    if args.workload in pf:
        return bench_prefill(args, pf[args.workload])
    cfg = config_by_name(args.workload)
    if isinstance(cfg, PrefixSharedConfig):
        return bench_prefix_shared(args, cfg)
    if args.gather_probe:
        return bench_gather_probe(args, cfg)
    sh = draw_decode_shapes(cfg)
    vals = draw_decode_values(cfg, sh.lens)
    B, Hq, H, d, dt = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.dtype
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]
    total = args.warmup + args.steps
    n_post = event_launches(args)  # per-launch event pass after the timed steps
    total_all = total + n_post
    grow = -(-total_all // args.replicas)  # tokens each replica appends
    stride = -(-(int(sh.lens.max()) + grow) // 16)
    # each replica's pool holds the batch plus its growth
    grow_blocks = B * (-(-grow // 16) + 1)
    nb = sh.num_blocks + grow_blocks
    order = np.concatenate([sh.free_order, np.arange(sh.num_blocks, nb, dtype=np.int32)])

    def dev_tensor(bits):
        a = np.ascontiguousarray(bits)
        t = torch.from_numpy(a.view(np.int16) if dt == "bf16" else a)
        return (t.view(torch.bfloat16) if dt == "bf16" else t).to("cuda")

    k_ctx, v_ctx, q_dev = dev_tensor(vals["k"]), dev_tensor(vals["v"]), dev_tensor(vals["q"])
    new_k = dev_tensor(draw_normal_storage((cfg.seed, 50), (total_all, B, H, d), dt))
    new_v = dev_tensor(draw_normal_storage((cfg.seed, 51), (total_all, B, H, d), dt))
    native = not (args.two_launch or args.separate_write or args.no_overlap)
    # fill mode is chosen inside the native stepper; the Python-driven paths
    # take the library default instead
    partition = args.partition if (native or args.partition >= 0) else 0
    reps = []
    for r in range(args.replicas):
        kc = torch.zeros((nb, H, 16, d), dtype=tdt, device="cuda")
        vc = torch.zeros_like(kc)
        pool = Pool(nb, H, d, dt, stride, 16, order, kc, vc)
        slots = np.concatenate([pool.alloc(int(L))[1] for L in sh.lens])
        pool.write_kv(k_ctx, v_ctx, torch.from_numpy(slots).cuda())
        it = DecodeIteration(pool, B, stride, Hq, partition, pipelined=not args.no_overlap)
        out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
        reps.append((pool, it, out, kc, vc))
    del k_ctx, v_ctx
    torch.cuda.synchronize()
    seqs = list(range(B))
    per_tok = 2 * H * d * cfg.elem_bytes

    ev = timing_events(n_post)
    span = timing_events(1)[0]
    step_bytes, infos = [], []

    seqs_np = np.arange(B, dtype=np.int32)
    ctx_tokens = [int(sh.lens.sum())] * args.replicas  # tokens in each replica before a step

    def step(s, evs=None):
        r = s % args.replicas
        pool, it, out, _, _ = reps[r]
        if native:
            lay = it.step(seqs_np, q_dev, out, new_k[s], new_v[s], cfg.scale, events=evs)
            info = lay.plan
        else:
            meta = it.prepare(seqs)
            it.launch(meta, q_dev, out, new_k[s], new_v[s], cfg.scale, events=evs,
                      fused=not (args.two_launch or args.separate_write),
                      fused_append=not args.separate_write)
            info = meta["info"]
        ctx_tokens[r] += B  # every sequence appended one token and attends over it
        step_bytes.append(ctx_tokens[r] * per_tok)
        infos.append(info)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    # the K timed steps carry no per-launch events (each costs the GPU ~5 us
    # around its dispatch); two events on the decode stream bracket them
    t0 = time.perf_counter()
    span[0].record()
    for s in range(args.warmup, total):
        step(s)
    span[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    span_ms = span[0].elapsed_time(span[1])
    # then n_post more steps with events attached to every decode dispatch:
    # each launch's own duration, for the spread and for comparison with a
    # profiler's kernel trace (not part of `value`)
    for k in range(n_post):
        step(total + k, ev[k])
    torch.cuda.synchronize()

    timed = range(args.warmup, total)
    kbytes = sum(step_bytes[s] for s in timed)
    mean_bytes = float(np.mean([step_bytes[s] for s in timed]))
    # average decode launch on the GPU over the timed steps: the span of the
    # decode stream / K, i.e. each launch's duration plus the idle gap before
    # the next dispatch (a conservative duration: the gap is counted)
    mean_kern_s = span_ms / 1e3 / args.steps
    achieved = mean_bytes / mean_kern_s / 1e9
    kern_ms = [ev[k][0].elapsed_time(ev[k][1]) for k in range(n_post)]
    post_bytes = float(np.mean([step_bytes[total + k] for k in range(n_post)]))
    timed_ctx = float(np.mean([step_bytes[s] for s in timed])) / per_tok / B
    value = kbytes / wall / 1e9
    info = infos[-1]
    # counter traffic per algorithmic byte of the committed profile, applied
    # to this line's bytes (taken while the kernel source is unchanged)
    ratio = committed_traffic_ratio(counter_summary(cfg.name)) if partition == -1 else None
    traffic = round(ratio * mean_bytes) if ratio else None
    res = {
        "metric": DECODE_METRICS.get(cfg.name, METRIC),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {"workload": cfg.name, "num_seqs": B, "num_q_heads": Hq, "num_kv_heads": H,
                   "head_dim": d, "block_size": 16, "mean_context": round(float(sh.lens.mean()), 1),
                   "mean_context_timed": round(timed_ctx, 1),
                   "max_context": int(sh.lens.max()), "partition_tokens": info.partition_tokens,
                   "partition_mode": {-1: "fill", 0: "default"}.get(partition, "fixed"),
                   "kv_loads": "cached" if info.shared_kv else "streaming",
                   "work_items": info.n_work, "replicas": args.replicas,
                   "decode_launches": 2 if args.two_launch else 1,
                   "new_kv_store": "write_kv" if args.separate_write else "in decode",
                   "upload": "compute stream" if args.no_overlap else "side stream",
                   "accumulate": "f32", "output": "f32"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "decode_tokens_per_s": round(B * args.steps / wall, 1),
        # one attention layer per step; a 32-layer model of this shape would
        # decode about 1/32 as many tokens per second (a projection)
        "decode_tokens_per_s_32_layer_projection": round(B * args.steps / wall / 32, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "traffic_ratio": round(ratio, 4) if ratio else None,
                     "kernel": decode_kernel_name(dt, d, Hq // H) + (" (partition kernel of two launches)"
                                                                     if args.two_launch else ""),
                     "kernel_ms_mean": round(mean_kern_s * 1e3, 5),
                     "timing": "HIP events on the decode stream around the K timed steps: span / K "
                               "(each launch plus the idle gap before the next dispatch)",
                     "timed_launches": args.steps,
                     "algorithmic_bytes_per_launch": int(mean_bytes),
                     "per_launch_events": {
                         "launches": n_post,
                         "kernel_ms_mean": round(float(np.mean(kern_ms)), 5),
                         "kernel_ms_median": round(float(np.median(kern_ms)), 5),
                         "kernel_ms_p10": round(float(np.percentile(kern_ms, 10)), 5),
                         "kernel_ms_p90": round(float(np.percentile(kern_ms, 90)), 5),
                         "algorithmic_bytes_per_launch": int(post_bytes),
                         "achieved": round(post_bytes / (float(np.mean(kern_ms)) / 1e3) / 1e9, 2),
                         "note": "the steps right after the timed ones, each decode dispatch carrying "
                                 "its own start/stop events (the kernel alone)"},
                     "kernel_source_sha": kernel_source_sha()},
    }
    for pool, it, *_ in reps:
        it.close()
        pool.close()
    del reps
    torch.cuda.empty_cache()
    res["copy_probe"] = copy_probe()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, sh, vals, -(-int(sh.lens.max()) // 16), args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
