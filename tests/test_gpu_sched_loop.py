"""GPU parity of scheduler-driven mixed iterations (prefill chunks + decode).

A seeded request stream runs through the library scheduler; each iteration's
items drive the device: the prefill slices' K/V go in with write_kv and one
pkv_paged_prefill launch computes their queries; the decoding sequences run
one pkv_paged_decode launch that stores each new token's K/V itself.  The
oracle scheduler (same decisions, checked equal) drives a mirrored host pool
with the same rows, and every output of every iteration is compared with
the float64 oracle (prefill: causal attention of the slice; decode: the
sequence's full context).  The small pool forces preemptions, so freed
blocks are reused and recomputed sequences rewrite their K/V; shared
prefixes are forked.  Decode launches alternate the two K/V load policies
(the plan's shared_kv hint).  The whole pool is free at the end.
"""

import numpy as np
import pytest
import torch

from oracle.allocator import OracleAllocator
from oracle.attention import decode_attention, prefill_attention, storage_to_f64
from oracle.kvcache import MirrorPool
from oracle.scheduler import OracleRequest, OracleScheduler
from paged_kv_cache_257_amd import Pool, decode_plan, decode_workspace_bytes, prefill_plan
from paged_kv_cache_257_amd.sched import Scheduler
from tests.gpu_helpers import TOL, TORCH_DTYPE, sync, to_device
from workloads import STORAGE_NUMPY, draw_normal_storage
from workloads.requests import draw_request_trace

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DT, HQ, HKV, D = "bf16", 8, 2, 128
SCALE = 1.0 / np.sqrt(D)


def test_scheduler_drives_prefill_and_decode():
    reqs = draw_request_trace(24, 12, rate=1.5, prompt_hi=300, mean_output=30, max_output=60,
                              prefix_len=64, n_prefixes=1, prefix_share=0.5)
    blocks, width = 90, 24
    order = np.random.default_rng(5).permutation(blocks).astype(np.int32)
    # per-request values for every position it will ever hold
    vals = []
    for i, r in enumerate(reqs):
        n = r["prompt_len"] + r["output_len"]
        vals.append(tuple(draw_normal_storage((77, 1000 + i, j), (n, h, D), DT)
                          for j, h in ((1, HQ), (2, HKV), (3, HKV))))
    # requests sharing a prefix id carry identical prefix K/V (they share the blocks)
    first = {}
    for i, r in enumerate(reqs):
        if r["prefix_id"] >= 0:
            f = first.setdefault(r["prefix_id"], i)
            for a, b in zip(vals[i][1:], vals[f][1:]):
                a[:r["prefix_len"]] = b[:r["prefix_len"]]
    shape = (blocks, HKV, 16, D)
    kc = torch.zeros(shape, dtype=TORCH_DTYPE[DT], device="cuda")
    vc = torch.zeros_like(kc)
    pool = Pool(blocks, HKV, D, DT, width, 16, order, kc, vc)
    sch = Scheduler(pool, reqs, 256, 64, 12)
    ora = OracleScheduler(OracleAllocator(blocks, 16, width, order), 256, 64, 12,
                          [OracleRequest(**r) for r in reqs])
    mirror = MirrorPool(blocks, HKV, D, STORAGE_NUMPY[DT], 16)
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    worst, steps, n_dec, n_pre = 0.0, 0, 0, 0
    try:
        while not ora.done():
            items, _ = sch.step()
            o_items, _ = ora.step()
            assert items == o_items, steps
            cow = pool.take_cow()
            assert [tuple(x) for x in cow.tolist()] == ora.a.take_cow()
            if len(cow):
                pool.copy_blocks(torch.from_numpy(np.ascontiguousarray(cow)).cuda())
                mirror.copy_blocks([tuple(x) for x in cow.tolist()])
            pre = [it for it in items if it[2] == 0]
            dec = [it for it in items if it[2] == 1]
            # prefill slices: write their K/V, then one launch
            if pre:
                qs, ks, vs, slots, q_lens, lens, seqs = [], [], [], [], [], [], []
                for i, seq, _, pos, n in pre:
                    table = pool.table(seq)
                    sl = np.array([table[p // 16] * 16 + p % 16 for p in range(pos, pos + n)], np.int64)
                    q, k, v = vals[i]
                    qs.append(q[pos:pos + n]); ks.append(k[pos:pos + n]); vs.append(v[pos:pos + n])
                    slots.append(sl); q_lens.append(n); lens.append(pos + n); seqs.append(seq)
                    mirror.write_kv(k[pos:pos + n], v[pos:pos + n], sl)
                pool.write_kv(to_device(np.concatenate(ks), DT), to_device(np.concatenate(vs), DT),
                              torch.from_numpy(np.concatenate(slots)).cuda())
                tables, blens = pool.build_batch(seqs, width)
                assert blens.tolist() == lens
                plan, info = prefill_plan(q_lens, lens, HQ, HKV)
                out = torch.empty((sum(q_lens), HQ, D), dtype=torch.float32, device="cuda")
                pool.paged_prefill(to_device(np.concatenate(qs), DT), out, torch.from_numpy(tables).cuda(),
                                   torch.from_numpy(blens).cuda(), SCALE, torch.from_numpy(plan).cuda(), info)
                sync()
                got = out.cpu().numpy().astype(np.float64)
                off = 0
                for (i, seq, _, pos, n) in pre:
                    K, V = mirror.gather(ora.a.table(seq), pos + n)
                    ref = prefill_attention(storage_to_f64(vals[i][0][pos:pos + n], DT),
                                            storage_to_f64(K, DT), storage_to_f64(V, DT), SCALE)
                    err = float(np.max(np.abs(got[off:off + n] - ref)))
                    worst = max(worst, err)
                    assert err <= TOL[DT], (steps, i, pos, n, err)
                    off += n
                    n_pre += n
            # decode: the new token's K/V are stored by the decode launch itself
            if dec:
                seqs = [seq for _, seq, _, _, _ in dec]
                tables, lens = pool.build_batch(seqs, width)
                q = np.stack([vals[i][0][pos] for i, _, _, pos, _ in dec])
                kn = np.stack([vals[i][1][pos] for i, _, _, pos, _ in dec])
                vn = np.stack([vals[i][2][pos] for i, _, _, pos, _ in dec])
                for (i, seq, _, pos, _), k1, v1 in zip(dec, kn, vn):
                    table = ora.a.table(seq)
                    mirror.write_kv(k1[None], v1[None], np.array([table[pos // 16] * 16 + pos % 16]))
                plan, info = decode_plan(lens, 0)
                assert pool.batch_shared_kv(seqs) in (0, 1)
                info.shared_kv = steps % 2  # both load policies, alternately
                assert decode_workspace_bytes(info, HQ, D) <= ws.numel()
                out = torch.empty((len(dec), HQ, D), dtype=torch.float32, device="cuda")
                pool.paged_decode(to_device(q, DT), out, torch.from_numpy(tables).cuda(),
                                  torch.from_numpy(lens).cuda(), SCALE, torch.from_numpy(plan).cuda(), info,
                                  ws, k_new=to_device(kn, DT), v_new=to_device(vn, DT))
                sync()
                got = out.cpu().numpy().astype(np.float64)
                for j, (i, seq, _, pos, _) in enumerate(dec):
                    K, V = mirror.gather(ora.a.table(seq), pos + 1)
                    ref = decode_attention(storage_to_f64(q[j], DT), storage_to_f64(K, DT),
                                           storage_to_f64(V, DT), SCALE)
                    err = float(np.max(np.abs(got[j] - ref)))
                    worst = max(worst, err)
                    assert err <= TOL[DT], (steps, i, pos, err)
                n_dec += len(dec)
            steps += 1
            assert steps < 5000
        assert sch.step()[0] == ora.step()[0] == []  # frees the last finished sequences
        st = sch.stats()
        assert st["preemptions"] > 0 and st["prefix_hit_tokens"] > 0
        assert pool.stats()["free_blocks"] == blocks
        print(f"\n[gpu] scheduler loop: {steps} iterations, {n_pre} prefill tokens, {n_dec} decodes, "
              f"{st['preemptions']} preemptions, {st['prefix_hit_tokens']} prefix-hit tokens, "
              f"max_err={worst:.3e}", flush=True)
    finally:
        sch.close()
        pool.close()
