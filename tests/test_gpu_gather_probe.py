"""GPU: the gather probe (pkv_gather_probe) reads exactly the tiles a decode
plan makes the decode read.

Each wave's output is the XOR of every 32-bit word of the K and V tiles of
its blocks; the host computes the same from the pool's bits and the plan's
work list.  Bit-exact for every staging mode and wave count, on ragged
batches (a one-token sequence, partial last blocks, several partitions and
64-entry table chunks), on 2 KiB, 4 KiB and 8 KiB tiles; the LDS mode
refuses tiles over 4 KiB.
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_257_amd import PkvError, Pool, decode_plan

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def expected(kw, vw, tables, lens, plan, info, H, waves):
    """[n_work][H][waves] XOR of the words of each wave's K and V tiles."""
    pb = info.partition_tokens // 16
    out = np.zeros((info.n_work, H, waves), np.uint32)
    for wi in range(info.n_work):
        seq, part = int(plan[2 * wi]), int(plan[2 * wi + 1])
        nblk = min(-(-int(lens[seq]) // 16), tables.shape[1])
        b0, b1 = part * pb, min(part * pb + pb, nblk)
        for w in range(waves):
            blks = tables[seq, b0 + w:b1:waves]
            if len(blks) == 0:
                continue
            x = np.bitwise_xor.reduce(kw[blks].reshape(len(blks), H, -1), axis=(0, 2)) ^ \
                np.bitwise_xor.reduce(vw[blks].reshape(len(blks), H, -1), axis=(0, 2))
            out[wi, :, w] = x
    return out


@pytest.mark.parametrize("dtype,head_dim,H", [("f16", 128, 4), ("bf16", 64, 2), ("f32", 128, 2)])
@pytest.mark.parametrize("partition", [0, 256])
def test_probe_reads_the_plans_tiles(dtype, head_dim, H, partition):
    rng = np.random.default_rng(7)
    lens = np.array([1, 17, 1500, 1024, 33, 2100, 16, 300], dtype=np.int64)
    width = -(-int(lens.max()) // 16)
    num_blocks = int(sum(-(-int(L) // 16) for L in lens)) + 11
    order = rng.permutation(num_blocks).astype(np.int32)
    shape = (num_blocks, H, 16, head_dim)
    words = num_blocks * H * 16 * head_dim * (4 if dtype == "f32" else 2) // 4
    kw = rng.integers(0, 2**32, size=words, dtype=np.uint32)
    vw = rng.integers(0, 2**32, size=words, dtype=np.uint32)
    k_cache = torch.from_numpy(kw.view(np.int32)).cuda().view(TORCH_DTYPE[dtype]).view(shape)
    v_cache = torch.from_numpy(vw.view(np.int32)).cuda().view(TORCH_DTYPE[dtype]).view(shape)
    pool = Pool(num_blocks, H, head_dim, dtype, width, 16, order, k_cache, v_cache)
    try:
        seqs = [pool.alloc(int(L))[0] for L in lens]
        tables, clens = pool.build_batch(seqs, width)
        plan, info = decode_plan(clens, partition)
        assert info.n_work > len(lens) or partition == 0
        t_d, l_d, p_d = (torch.from_numpy(a).cuda() for a in (tables, clens, plan))
        kw_b = kw.reshape(num_blocks, -1)
        vw_b = vw.reshape(num_blocks, -1)
        modes = ["regs", "cached"] + (["lds"] if 16 * head_dim * (4 if dtype == "f32" else 2) <= 4096 else [])
        for waves in (1, 2, 4):
            exp = expected(kw_b, vw_b, tables, clens, plan, info, H, waves)
            for mode in modes:
                out = torch.full((info.n_work * H * waves,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
                pool.gather_probe(t_d, l_d, p_d, info, out, mode, waves)
                torch.cuda.synchronize()
                got = out.cpu().numpy().view(np.uint32).reshape(info.n_work, H, waves)
                assert np.array_equal(got, exp), (mode, waves)
        if "lds" not in modes:
            out = torch.zeros(info.n_work * H * 4, dtype=torch.int32, device="cuda")
            with pytest.raises(PkvError):
                pool.gather_probe(t_d, l_d, p_d, info, out, "lds", 4)
    finally:
        pool.close()
        del k_cache, v_cache
        torch.cuda.empty_cache()
