"""GPU: the native stepper in fill mode (partition_tokens = PKV_PARTITION_FILL).

Each iteration the stepper picks the smallest split-K partition whose
workgroups are all resident at once (pkv_decode_fill_partition over the
device occupancy pkv_decode_occupancy reports), else the default.  Checked:
the partition it used equals that rule applied to the batch's lengths after
the append, and the outputs of the appending decode match the oracle over
the same logical tokens (max |err| <= 2e-3, fp32 accumulation).  One batch
where the rule picks a size (grouped queries, a few long sequences) and one
where nothing fits and the default is kept (many short MHA sequences).
Each batch runs with the upload on a copy stream of its own and, without
one, on the compute stream.
"""

import dataclasses

import numpy as np
import pytest
import torch

from oracle.runs import DecodeRun
from paged_kv_cache_257_amd import Pool, default_partition_tokens, fill_partition
from paged_kv_cache_257_amd.step import PARTITION_FILL, DecodeIteration
from tests.gpu_helpers import TOL, TORCH_DTYPE, sync, to_device
from workloads import config_by_name, draw_decode_values

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CASES = {
    # grouped queries, long sequences: the rule picks a partition
    "gqa_long": (dict(dtype="bf16", num_q_heads=32, num_kv_heads=8),
                 [9000, 3001, 7777, 100, 16, 17]),
    # MHA, 64 short sequences x 32 heads: nothing fits one round, default kept
    "mha_short": (dict(dtype="f16", num_q_heads=32, num_kv_heads=32),
                  list(np.random.default_rng(3).integers(1, 1500, size=64))),
}


@pytest.mark.parametrize("pipelined", [True, False], ids=["copy_stream", "compute_stream"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_stepper_fill_mode(name, pipelined):
    over, lens = CASES[name]
    lens = np.asarray(lens, dtype=np.int64)
    cfg = dataclasses.replace(config_by_name("gpt_f16"), name="fill_" + name, index=500 + len(name), head_dim=128,
                              num_seqs=len(lens), **over)
    H, d, dt, Hq = cfg.num_kv_heads, cfg.head_dim, cfg.dtype, cfg.num_q_heads
    nb = int(sum(-(-int(L) // 16) for L in lens)) + 4
    order = np.random.default_rng(cfg.index).permutation(nb).astype(np.int32)
    stride = max(-(-int(L) // 16) for L in lens)
    vals = draw_decode_values(cfg, lens)
    ora = DecodeRun(cfg, lens, nb, order, stride)
    ora.write_context(vals["k"], vals["v"])
    k_cache = torch.full((nb, H, 16, d), float("nan"), dtype=TORCH_DTYPE[dt], device="cuda")
    v_cache = torch.full_like(k_cache, float("nan"))
    pool = Pool(nb, H, d, dt, stride, 16, order, k_cache, v_cache)
    try:
        # the pool holds every token but each sequence's newest; the stepper
        # appends it (k_new / v_new) and attends over all of them
        last = np.cumsum(lens) - 1
        keep = np.ones(int(lens.sum()), dtype=bool)
        keep[last] = False
        slots = np.concatenate([pool.alloc(int(L) - 1)[1] for L in lens])
        pool.write_kv(to_device(np.ascontiguousarray(vals["k"][keep]), dt),
                      to_device(np.ascontiguousarray(vals["v"][keep]), dt), torch.from_numpy(slots).cuda())
        wpi, resident = pool.decode_occupancy(Hq)
        assert wpi >= 1 and resident >= 1
        want = fill_partition(lens, wpi, resident, 512) or default_partition_tokens()
        print(f"\n[gpu] fill {name} pipelined={pipelined}: workgroups/item={wpi} resident={resident} "
              f"-> P={want}", flush=True)
        step = DecodeIteration(pool, len(lens), stride, Hq, PARTITION_FILL, pipelined=pipelined)
        out = torch.full((len(lens), Hq, d), float("nan"), dtype=torch.float32, device="cuda")
        meta = step.step(list(range(len(lens))), to_device(vals["q"], dt), out,
                         to_device(np.ascontiguousarray(vals["k"][last]), dt),
                         to_device(np.ascontiguousarray(vals["v"][last]), dt), cfg.scale, host_meta=True)
        sync()
        assert meta["info"].partition_tokens == want
        got = out.cpu().numpy().astype(np.float64)
        err = max(float(np.max(np.abs(got[i] - ora.attend(i, vals["q"][i])))) for i in range(len(lens)))
        print(f"[gpu] fill {name}: work={meta['info'].n_work} max_err={err:.3e}", flush=True)
        assert np.isfinite(got).all() and err <= TOL[dt]
        step.close()
        if name == "gqa_long":
            assert want != default_partition_tokens()
        else:
            assert want == default_partition_tokens()
    finally:
        pool.close()
        del k_cache, v_cache
        torch.cuda.empty_cache()
