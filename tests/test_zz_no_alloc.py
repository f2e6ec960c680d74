"""GPU test of pkv_paged_decode_noalloc, the decode entry point for callers
that cannot allocate device memory: its output must equal pkv_paged_decode's
bit for bit (the same kernels on the same inputs; only where the split-K
records live differs), and the oracle's within the workload tolerance, on
two calls in a row with the second batch smaller than the first, so that
the second runs over scratch the first has left records and tickets in.
A batch that needs more scratch than the library holds is refused before
any launch."""

import dataclasses

import numpy as np
import pytest
import torch

from paged_kv_cache_257_amd import PkvError, decode_plan, decode_workspace_bytes
from paged_kv_cache_257_amd import _capi
from tests.gpu_helpers import TOL, DecodeCase, sync, to_device
from workloads import config_by_name

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _cases():
    # (workload, lengths, partition tokens): the second of each pair is the
    # smaller batch; small partitions so that every call writes split-K
    # records and takes tickets
    mha = dataclasses.replace(config_by_name("gpt_f16"), name="noalloc_mha", index=60)
    gqa = dataclasses.replace(config_by_name("gqa_long_bf16"), name="noalloc_gqa", index=61)
    rng = np.random.default_rng(61)
    big = [int(x) for x in rng.integers(1, 3000, size=40)] + [1, 16, 17, 2047]
    small = [5, 700, 33, 1500]
    return [(mha, big, 256), (mha, small, 128), (gqa, big, 512), (gqa, small, 64)]


def _run(cfg, lens, P):
    nb = sum(-(-L // 16) for L in lens) + 8
    case = DecodeCase(cfg, lens=lens, num_blocks=nb,
                      free_order=np.random.default_rng(len(lens)).permutation(nb), fill=float("nan"))
    try:
        case.write_context()
        ref_out, info = case.decode(P)  # pkv_paged_decode with a fresh zeroed workspace
        assert info.n_reduce > 0
        tables, lens_h = case.pool.build_batch(case.seqs, case.stride)
        plan, info = decode_plan(lens_h, P)
        q = to_device(case.vals["q"], cfg.dtype)
        out = torch.full((len(lens), cfg.num_q_heads, cfg.head_dim), float("nan"),
                         dtype=torch.float32, device="cuda")
        print(f"[gpu] noalloc {cfg.name} B={len(lens)} P={P} work={info.n_work} reduce={info.n_reduce}",
              flush=True)
        case.pool.paged_decode_noalloc(q, out, torch.from_numpy(tables).cuda(),
                                       torch.from_numpy(lens_h).cuda(), cfg.scale,
                                       torch.from_numpy(plan).cuda(), info)
        sync()
        got = out.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref_out)  # bit for bit the workspace entry point's
        err = float(np.max(np.abs(got - case.oracle_all())))
        assert err <= TOL[cfg.dtype], err
    finally:
        case.close()


def test_noalloc_matches_workspace_decode_twice():
    cases = _cases()
    for cfg, lens, P in cases:
        _run(cfg, lens, P)


def test_noalloc_refuses_batches_beyond_its_scratch():
    cfg = config_by_name("gpt_f16")
    lens = np.full(512, 8192, dtype=np.int32)
    plan, info = decode_plan(lens, 16)
    need = decode_workspace_bytes(info, cfg.num_q_heads, cfg.head_dim)
    assert need > _capi.NOALLOC_SCRATCH_BYTES
    case = DecodeCase(dataclasses.replace(cfg, index=62), lens=[1], num_blocks=2, free_order=[1, 0])
    try:
        q = torch.zeros((512, cfg.num_q_heads, cfg.head_dim), dtype=torch.float16, device="cuda")
        out = torch.zeros((512, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
        tb = torch.zeros((512, 512), dtype=torch.int32, device="cuda")
        with pytest.raises(PkvError) as e:
            case.pool.paged_decode_noalloc(q, out, tb, torch.from_numpy(lens).cuda(), cfg.scale,
                                           torch.from_numpy(plan).cuda(), info)
        assert e.value.status == _capi.E_BAD_ARG and "scratch" in str(e.value)
        sync()
    finally:
        case.close()
