"""GPU parity: write_kv, copy_blocks and paged_decode against the oracle.

* every decode workload at its full size: block tables and slots bit-exact,
  the whole written pool bit-exact, and the attention output of every
  sequence and head within the tolerance the workload states: max |err|
  <= 1e-5 for fp32 inputs, <= 2e-3 for fp16/bf16 (fp32 accumulation, fp32
  output);
* each at the partition size the benchmark uses, at a second one and at the
  one fill mode picks, so both the single-partition and the split-K + reduce
  paths are compared;
* masking: pools pre-filled with NaN must not leak into outputs;
* a sweep over dtypes, head dims 64/128/256, GQA groups 1-8 and ragged
  lengths around block boundaries (1, 15, 16, 17, ...);
* copy-on-write block copies bit-exact against the mirrored pool.
"""

import dataclasses

import numpy as np
import pytest
import torch

from paged_kv_cache_257_amd import default_partition_tokens, fill_partition
from tests.gpu_helpers import TOL, DecodeCase, device_bits, host_bits, peaked_qk, sync, to_device
from workloads import CONFIGS, config_by_name, draw_decode_values, draw_normal_storage
from workloads.configs import DecodeConfig

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# partition sizes: the one the benchmark times first, then another
PARTITIONS = {"tiny_f32": (0, 16), "gpt_f16": (0, 2048), "ragged_bf16": (0, 512),
              "gqa_long_bf16": (512, 0)}


def max_err(case, out, seqs):
    worst = 0.0
    for i in seqs:
        worst = max(worst, float(np.max(np.abs(out[i] - case.oracle_out(i)))))
    return worst


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_workload_parity(cfg):
    print(f"\n[gpu] workload {cfg.name}", flush=True)
    case = DecodeCase(cfg)
    try:
        t_c, l_c = case.pool.build_batch(case.seqs, case.stride)
        t_o, l_o = case.oracle.tables(case.stride)
        assert np.array_equal(t_c, np.asarray(t_o, np.int32))
        assert np.array_equal(l_c, np.asarray(l_o, np.int32))
        assert np.array_equal(case.slots, case.oracle.slots)
        case.write_context()
        assert np.array_equal(device_bits(case.k_cache), host_bits(case.oracle.mirror.k))
        assert np.array_equal(device_bits(case.v_cache), host_bits(case.oracle.mirror.v))
        ref = case.oracle_all()  # every sequence
        # and the partition fill mode picks for this batch (the bench's default)
        wpi, resident = case.pool.decode_occupancy(cfg.num_q_heads)
        p_fill = fill_partition(case.lens, wpi, resident, 512) or default_partition_tokens()
        for P in PARTITIONS[cfg.name] + (p_fill,):
            for split in (False, True):
                out, info = case.decode(P, split=split)
                err = float(np.max(np.abs(out - ref)))
                print(f"[gpu] {cfg.name} P={info.partition_tokens} split={split} work={info.n_work} "
                      f"reduce={info.n_reduce} max_err={err:.3e}", flush=True)
                assert err <= TOL[cfg.dtype], (P, split, err)
                assert np.isfinite(out).all()
                assert case.last_tickets_zero
    finally:
        case.close()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_nan_filled_pool_does_not_leak(dtype):
    cfg = dataclasses.replace(config_by_name("tiny_f32"), dtype=dtype, index=20, head_dim=128 if dtype != "f32" else 64)
    lens = [1, 5, 16, 17, 31, 33, 60]
    order = np.random.default_rng(7).permutation(40)
    case = DecodeCase(cfg, lens=lens, num_blocks=40, free_order=order, fill=float("nan"))
    try:
        case.write_context()
        for P in (16, 0):
            out, _ = case.decode(P)
            assert np.isfinite(out).all()
            assert max_err(case, out, range(len(lens))) <= TOL[dtype]
    finally:
        case.close()


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_fused_append_decode(cfg):
    """k_new/v_new path: the pool holds every token but each sequence's newest;
    one launch stores the newest rows and attends over all of them (at the
    bench's first partition size and at the one fill mode picks)."""
    print(f"\n[gpu] append-decode {cfg.name}", flush=True)
    case = DecodeCase(cfg, fill=float("nan"))
    try:
        case.write_context(skip_last=True)
        ref = case.oracle_all()  # every sequence
        wpi, resident = case.pool.decode_occupancy(cfg.num_q_heads)
        p_fill = fill_partition(case.lens, wpi, resident, 512) or default_partition_tokens()
        for P in (PARTITIONS[cfg.name][0], p_fill):
            out, info = case.decode(P, append=True)
            err = float(np.max(np.abs(out - ref)))
            print(f"[gpu] append-decode {cfg.name} P={info.partition_tokens} max_err={err:.3e}", flush=True)
            assert err <= TOL[cfg.dtype] and np.isfinite(out).all()
        # the newest rows landed in the pool: bit-exact everywhere a token lives
        kd, vd = device_bits(case.k_cache), device_bits(case.v_cache)
        km, vm = host_bits(case.oracle.mirror.k), host_bits(case.oracle.mirror.v)
        s = case.slots
        blk, row = s // 16, s % 16
        assert np.array_equal(kd[blk, :, row, :], km[blk, :, row, :])
        assert np.array_equal(vd[blk, :, row, :], vm[blk, :, row, :])
    finally:
        case.close()


@pytest.mark.parametrize("group,q_heads", [(1, 4), (6, 6), (12, 24), (16, 16)])
def test_fused_append_decode_gqa_groups(group, q_heads):
    """Several workgroups (query-head groups) read the same new row; one stores it."""
    kv = q_heads // group
    cfg = dataclasses.replace(config_by_name("ragged_bf16"), name="append_gqa", index=40 + group, num_kv_heads=kv,
                              num_q_heads=kv * group, dtype="bf16")
    lens = [1, 2, 16, 17, 31, 100, 513, 700]
    nb = sum(-(-L // 16) for L in lens) + 2
    case = DecodeCase(cfg, lens=lens, num_blocks=nb, free_order=np.random.default_rng(group).permutation(nb),
                      fill=float("nan"))
    try:
        case.write_context(skip_last=True)
        for P in (16, 0):
            for split in (False, True):
                out, _ = case.decode(P, split=split, append=True)
                err = max_err(case, out, range(len(lens)))
                assert err <= TOL["bf16"], (P, split, err)
        kd = device_bits(case.k_cache)
        km = host_bits(case.oracle.mirror.k)
        blk, row = case.slots // 16, case.slots % 16
        assert np.array_equal(kd[blk, :, row, :], km[blk, :, row, :])
    finally:
        case.close()


SWEEP = [(dt, d, hkv, g) for dt in ("f32", "f16", "bf16") for d in (64, 128, 256)
         for hkv, g in ((2, 1), (2, 2), (1, 4), (2, 8))]


@pytest.mark.parametrize("dtype,head_dim,kv_heads,group", SWEEP)
def test_shape_sweep(dtype, head_dim, kv_heads, group):
    idx = 100 + SWEEP.index((dtype, head_dim, kv_heads, group))
    cfg = dataclasses.replace(config_by_name("tiny_f32"), name="sweep", index=idx, dtype=dtype, head_dim=head_dim,
                              num_kv_heads=kv_heads, num_q_heads=kv_heads * group, num_seqs=9)
    lens = [1, 15, 16, 17, 47, 64, 100, 129, 300]
    nb = sum(-(-L // 16) for L in lens) + 5
    order = np.random.default_rng(idx).permutation(nb)
    case = DecodeCase(cfg, lens=lens, num_blocks=nb, free_order=order)
    try:
        case.write_context()
        for P in (16, 64, 0):
            for split in (False, True):
                out, _ = case.decode(P, split=split)
                err = max_err(case, out, range(len(lens)))
                assert err <= TOL[dtype], (P, split, err)
                assert case.last_tickets_zero
    finally:
        case.close()


def test_copy_blocks_bit_exact():
    cfg = dataclasses.replace(config_by_name("gpt_f16"), index=30, num_seqs=1)
    nb, H, d = 64, cfg.num_kv_heads, cfg.head_dim
    case = DecodeCase(cfg, lens=[nb * 16], num_blocks=nb, free_order=np.arange(nb))
    try:
        case.write_context()
        rng = np.random.default_rng(3)
        blocks = rng.permutation(nb)
        pairs = np.stack([blocks[:12], blocks[12:24]], axis=1).astype(np.int32)
        case.pool.copy_blocks(torch.from_numpy(pairs).cuda())
        sync()
        case.oracle.mirror.copy_blocks([tuple(p) for p in pairs.tolist()])
        assert np.array_equal(device_bits(case.k_cache), host_bits(case.oracle.mirror.k))
        assert np.array_equal(device_bits(case.v_cache), host_bits(case.oracle.mirror.v))
    finally:
        case.close()


def test_write_kv_skips_negative_and_out_of_pool_slots():
    cfg = dataclasses.replace(config_by_name("tiny_f32"), index=31)
    case = DecodeCase(cfg, lens=[32], num_blocks=4, free_order=np.arange(4))
    try:
        case.write_context()
        k = draw_normal_storage((5, 1), (4, cfg.num_kv_heads, cfg.head_dim), "f32")
        slots = np.array([3, -1, 64, -7], dtype=np.int64)  # pool holds slots 0..63
        case.pool.write_kv(to_device(k, "f32"), to_device(k, "f32"), torch.from_numpy(slots).cuda())
        sync()
        keep = (slots >= 0) & (slots < 64)
        case.oracle.mirror.write_kv(k[keep], k[keep], slots[keep])
        assert np.array_equal(device_bits(case.k_cache), host_bits(case.oracle.mirror.k))
        assert np.array_equal(device_bits(case.v_cache), host_bits(case.oracle.mirror.v))
    finally:
        case.close()


def test_workspace_shared_by_launches_of_different_shapes():
    """One workspace sized by pkv_decode_workspace_bound serves, in turn, a
    batch of 2 long sequences (many split-K records) and a batch of 40
    shorter ones (more completion tickets), twice: records grow from the
    workspace's start and tickets sit at its end, so neither launch sees the
    other's leftovers."""
    from paged_kv_cache_257_amd import decode_workspace_bound
    base = dataclasses.replace(config_by_name("gpt_f16"), name="shared_ws", index=60, dtype="bf16", num_kv_heads=8,
                               num_q_heads=32)
    long_lens = [3000, 2500]
    short_lens = [int(x) for x in np.random.default_rng(60).integers(100, 2500, size=40)]
    cases = []
    for lens in (long_lens, short_lens):
        cfg = dataclasses.replace(base, num_seqs=len(lens))
        nb = sum(-(-L // 16) for L in lens) + 3
        cases.append(DecodeCase(cfg, lens=lens, num_blocks=nb,
                                free_order=np.random.default_rng(len(lens)).permutation(nb)))
        cases[-1].write_context()
    try:
        ws_bytes = decode_workspace_bound(40, 3000, 32, 128, 512)
        workspace = torch.zeros(ws_bytes // 4, dtype=torch.float32, device="cuda")
        for rnd in range(2):
            for case in cases:
                got, info = case.decode(512, workspace=workspace)
                assert info.n_partials > 0
                err = max(float(np.max(np.abs(got[i] - case.oracle_out(i)))) for i in range(len(case.lens)))
                print(f"[gpu] shared workspace round {rnd} batch {len(case.lens)}: max_err={err:.3e}", flush=True)
                assert err <= TOL["bf16"], err
                assert case.last_tickets_zero
    finally:
        for case in cases:
            case.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("group", [2, 4, 8, 16])
def test_gqa_both_kernels(dtype, group, monkeypatch):
    """Grouped-query decode of head_dim 128 runs on the matrix-core kernel by
    default; PKV_DECODE_MFMA=0 selects the VALU kernel.  Both against the
    oracle, with and without the fused append, split and unsplit."""
    idx = 300 + 10 * group + (dtype == "bf16")
    cfg = dataclasses.replace(config_by_name("tiny_f32"), name="gqa_kernels", index=idx, dtype=dtype, head_dim=128,
                              num_kv_heads=2, num_q_heads=2 * group, num_seqs=10)
    lens = [1, 2, 15, 16, 17, 33, 100, 257, 600, 1111]
    nb = sum(-(-L // 16) for L in lens) + 3
    order = np.random.default_rng(idx).permutation(nb)
    case = DecodeCase(cfg, lens=lens, num_blocks=nb, free_order=order, fill=float("nan"))
    try:
        case.write_context(skip_last=True)
        for mode in ("1", "0"):
            monkeypatch.setenv("PKV_DECODE_MFMA", mode)
            for P in (16, 256, 0):
                for split in (False, True):
                    out, _ = case.decode(P, split=split, append=True)
                    err = max_err(case, out, range(len(lens)))
                    print(f"[gpu] gqa {dtype} group={group} mfma={mode} P={P} split={split} "
                          f"max_err={err:.3e}", flush=True)
                    assert np.isfinite(out).all()
                    assert err <= TOL[dtype], (mode, P, split, err)
                    assert case.last_tickets_zero
    finally:
        case.close()


@pytest.mark.parametrize("dtype,group", [("f16", 1), ("bf16", 1), ("f32", 2), ("bf16", 4), ("f16", 8)])
def test_tuning_variants(dtype, group, monkeypatch):
    """Every decode variant the tuning variables reach (waves per workgroup
    1/2/4/8, query heads per workgroup capped at 1/2/4, either kernel for
    grouped queries) against the oracle, with the fused append, split and
    unsplit: they are read at every launch."""
    idx = 400 + 10 * group + {"f32": 0, "f16": 1, "bf16": 2}[dtype]
    d = 64 if dtype == "f32" else 128
    cfg = dataclasses.replace(config_by_name("tiny_f32"), name="tuning", index=idx, dtype=dtype, head_dim=d,
                              num_kv_heads=2, num_q_heads=2 * group, num_seqs=7)
    lens = [1, 16, 17, 40, 129, 300, 700]
    nb = sum(-(-L // 16) for L in lens) + 3
    case = DecodeCase(cfg, lens=lens, num_blocks=nb, free_order=np.random.default_rng(idx).permutation(nb),
                      fill=float("nan"))
    try:
        case.write_context(skip_last=True)
        for waves in ("1", "2", "4", "8"):
            for cap in ("16", "2", "1"):
                for mfma in ("1", "0"):
                    monkeypatch.setenv("PKV_DECODE_WAVES", waves)
                    monkeypatch.setenv("PKV_DECODE_GW", cap)
                    monkeypatch.setenv("PKV_DECODE_MFMA", mfma)
                    for P in (64, 0):
                        out, _ = case.decode(P, split=(P == 64 and waves == "2"), append=True)
                        err = max_err(case, out, range(len(lens)))
                        assert np.isfinite(out).all(), (waves, cap, mfma, P)
                        assert err <= TOL[dtype], (waves, cap, mfma, P, err)
                        assert case.last_tickets_zero
    finally:
        case.close()


@pytest.mark.parametrize("dtype,group", [("f32", 1), ("f16", 1), ("bf16", 1), ("bf16", 4), ("f16", 8)])
def test_cached_tile_loads(dtype, group, monkeypatch):
    """The plan's load-policy hint (shared_kv = 1: tile loads through the
    caches, 4 waves per workgroup) gives bit for bit the output of the
    streaming loads at 4 waves, within the oracle's tolerance, for both
    kernels, split and unsplit, with the fused append."""
    idx = 600 + 10 * group + {"f32": 0, "f16": 1, "bf16": 2}[dtype]
    d = 64 if dtype == "f32" else 128
    cfg = dataclasses.replace(config_by_name("tiny_f32"), name="cached_loads", index=idx, dtype=dtype,
                              head_dim=d, num_kv_heads=2, num_q_heads=2 * group, num_seqs=7)
    lens = [1, 16, 17, 40, 129, 300, 700]
    nb = sum(-(-L // 16) for L in lens) + 3
    case = DecodeCase(cfg, lens=lens, num_blocks=nb, free_order=np.random.default_rng(idx).permutation(nb),
                      fill=float("nan"))
    try:
        case.write_context(skip_last=True)
        monkeypatch.setenv("PKV_DECODE_WAVES", "4")
        for mfma in (("1", "0") if group > 1 else ("0",)):
            monkeypatch.setenv("PKV_DECODE_MFMA", mfma)
            for P, split in ((64, False), (64, True), (0, False)):
                outs = []
                for shared in (0, 1):
                    out, info = case.decode(P, split=split, append=True, shared_kv=shared)
                    assert info.shared_kv == shared
                    assert np.isfinite(out).all(), (mfma, P, split, shared)
                    assert max_err(case, out, range(len(lens))) <= TOL[dtype], (mfma, P, split, shared)
                    assert case.last_tickets_zero
                    outs.append(out)
                assert np.array_equal(outs[0], outs[1]), (mfma, P, split)
    finally:
        case.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_lds_staged_variant(dtype, monkeypatch):
    """The LDS-staged instance of the VALU kernel (the default at 4 waves for
    fp16 / bf16, head_dim 128: tiles loaded straight into a per-wave LDS
    ring, read back into the same registers) gives bit for bit the output of
    the register-staged one (PKV_DECODE_STAGING=regs), within the oracle's
    tolerance, split and unsplit, with the fused append, over a NaN-filled
    pool and tables longer than one 64-entry chunk."""
    idx = 700 + {"f16": 1, "bf16": 2}[dtype]
    cfg = dataclasses.replace(config_by_name("tiny_f32"), name="lds_staged", index=idx, dtype=dtype,
                              head_dim=128, num_kv_heads=2, num_q_heads=2, num_seqs=8)
    lens = [1, 16, 17, 40, 129, 300, 1100, 2100]
    nb = sum(-(-L // 16) for L in lens) + 3
    case = DecodeCase(cfg, lens=lens, num_blocks=nb, free_order=np.random.default_rng(idx).permutation(nb),
                      fill=float("nan"))
    try:
        case.write_context(skip_last=True)
        monkeypatch.setenv("PKV_DECODE_WAVES", "4")
        for P, split in ((64, False), (64, True), (1024, True), (0, False)):
            outs = []
            for staging in ("regs", "lds"):
                monkeypatch.setenv("PKV_DECODE_STAGING", staging)
                out, _ = case.decode(P, split=split, append=True)
                err = max_err(case, out, range(len(lens)))
                print(f"[gpu] staging={staging} {dtype} P={P} split={split} max_err={err:.3e}", flush=True)
                assert np.isfinite(out).all(), (staging, P, split)
                assert err <= TOL[dtype], (staging, P, split, err)
                assert case.last_tickets_zero
                outs.append(out)
            assert np.array_equal(outs[0], outs[1]), (P, split)
    finally:
        case.close()


@pytest.mark.parametrize("dtype,hq,hkv", [("f16", 8, 2), ("f16", 4, 4), ("bf16", 8, 2)])
def test_dominant_keys_outside_first_lane_group(dtype, hq, hkv):
    """Decode rows dominated, by about 43 in base 2, by the keys at block
    row 5 (lanes 16..31 of the matrix-core score layout): the running
    maximum must cover every lane group or the fp16 weights overflow.  Every
    output, unsplit and split."""
    lens = (6, 21, 37, 100, 333, 517, 1000)
    cfg = DecodeConfig(name=f"peak_{dtype}_{hq}_{hkv}", index=40, dtype=dtype, num_seqs=len(lens),
                       num_q_heads=hq, num_kv_heads=hkv, head_dim=128, length_rule="fixed", fixed_lengths=lens)
    vals = draw_decode_values(cfg, lens)
    pos = np.concatenate([np.arange(L) for L in lens])
    vals["q"], vals["k"] = peaked_qk(vals["q"], vals["k"], pos, dtype, seed=3)
    case = DecodeCase(cfg, values=vals)
    try:
        case.write_context()
        ref = case.oracle_all()
        for P, split in [(0, False), (64, True), (512, False)]:
            out, _ = case.decode(P, split=split)
            err = float(np.max(np.abs(out - ref)))
            print(f"\n[gpu] peaked decode {dtype} {hq}/{hkv} P={P} split={split}: max err {err:.2e}", flush=True)
            assert np.isfinite(out).all() and err <= TOL[dtype], err
            assert case.last_tickets_zero
    finally:
        case.pool.close()

