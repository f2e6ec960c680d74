"""GPU parity of the shared-block decode: batches of forked sequences whose
common blocks are read once for all their holders (a separate launch writes
one split-K record per node chunk and member), then merged with each
sequence's own blocks.  Every output of every sequence and head is compared
with the oracle (fp64 attention over the blocks gathered through each
table) within 2e-3, for fp16 and bf16, MHA and grouped queries, several
chunk and partition sizes, the fused append of the newest token, the
two-launch variant, the no-allocation entry point, and pools whose unused
rows hold NaN.  The trees are built on the library allocator and on the
oracle allocator with the same operations; tables agree bit for bit."""

import dataclasses

import numpy as np
import pytest
import torch

from oracle.allocator import OracleAllocator
from oracle.attention import decode_attention, storage_to_f64
from paged_kv_cache_257_amd import Pool, decode_plan_shared, decode_workspace_bytes
from tests.gpu_helpers import TOL, TORCH_DTYPE, oracle_map, peaked_qk, sync, to_device
from workloads import draw_normal_storage

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

BS = 16


class ForkedCase:
    """A prompt shared by n_forks sequences with their own tails, plus
    forks of forks (lineages sharing tail blocks), one decode token
    appended to each; built identically on both allocators."""

    def __init__(self, seed, dtype="f16", kv_heads=4, group=1, prefix=1000, n_forks=48, tail_max=300,
                 lineages=16, nan_fill=True, peaked=False):
        rng = np.random.default_rng(seed)
        self.dtype, self.H, self.group, self.d = dtype, kv_heads, group, 128
        self.Hq = kv_heads * group
        need = -(-prefix // BS) + (n_forks + lineages) * (-(-(tail_max + 64) // BS) + 2)
        nb = int(need * 1.25) + 8
        # a lineage may fork a lineage: each link appends up to 40 tokens
        width = -(-(prefix + tail_max + 41 * (lineages + 1) + 16) // BS)
        order = rng.permutation(nb).astype(np.int32)
        self.k_cache = torch.zeros((nb, kv_heads, BS, 128), dtype=TORCH_DTYPE[dtype], device="cuda")
        self.v_cache = torch.zeros_like(self.k_cache)
        self.pool = Pool(nb, kv_heads, 128, dtype, width, BS, order, self.k_cache, self.v_cache)
        self.ora = OracleAllocator(nb, BS, width, order)
        root = self._both("alloc", prefix)
        seqs = []
        for _ in range(n_forks):
            c = self._both("fork", root)
            t = int(rng.integers(0, tail_max + 1))
            if t:
                self._both("append", c, t)
            seqs.append(c)
        for _ in range(lineages):
            c = self._both("fork", seqs[int(rng.integers(0, len(seqs)))])
            self._both("append", c, int(rng.integers(1, 40)))
            seqs.append(c)
        self._both("append_batch", seqs, 1)
        assert [tuple(p) for p in self.pool.take_cow().tolist()] == [tuple(p) for p in self.ora.take_cow()]
        self.seqs, self.width, self.nb = seqs, width, nb
        # pool contents: seeded values everywhere, NaN in the unused rows of
        # each last block (never attended)
        shape = (nb, kv_heads, BS, 128)
        kb = draw_normal_storage((seed, 1), shape, dtype)
        vb = draw_normal_storage((seed, 2), shape, dtype)
        q = draw_normal_storage((seed, 3), (len(seqs), self.Hq, 128), dtype)
        if peaked:  # every block's row 5 dominates (see peaked_qk)
            rows = np.ascontiguousarray(kb.transpose(0, 2, 1, 3)).reshape(nb * BS, kv_heads, 128)
            q, rows = peaked_qk(q, rows, np.tile(np.arange(BS), nb), dtype, seed)
            kb = np.ascontiguousarray(rows.reshape(nb, BS, kv_heads, 128).transpose(0, 2, 1, 3))
        if nan_fill:
            nan_bits = {"f16": np.float16(np.nan).view(np.uint16), "bf16": np.uint16(0x7FC0)}[dtype]
            for s in seqs:
                L, tab = self.ora.length(s), self.ora.table(s)
                if L % BS:
                    kb.view(np.uint16)[tab[-1], :, L % BS:, :] = nan_bits
                    vb.view(np.uint16)[tab[-1], :, L % BS:, :] = nan_bits
        self.kb, self.vb = kb, vb
        self.k_cache.copy_(to_device(kb, dtype))
        self.v_cache.copy_(to_device(vb, dtype))
        self.q = q
        tables, lens = self.pool.build_batch(seqs, width)
        t_o, l_o = self.ora.build_batch(seqs, width)
        assert np.array_equal(tables, np.asarray(t_o, np.int32)) and np.array_equal(lens, np.asarray(l_o))
        self.tables, self.lens = tables, lens
        sync()

    def _both(self, op, *args):
        a = getattr(self.pool, op)(*args)
        b = getattr(self.ora, op)(*args)
        if op == "alloc":
            assert a[0] == b[0]
            return a[0]
        if op == "fork":
            assert a == b
        return a

    def oracle_out(self, i):
        s = self.seqs[i]
        tab, L = np.asarray(self.ora.table(s)), self.ora.length(s)
        K = self.kb[tab].transpose(0, 2, 1, 3).reshape(-1, self.H, 128)[:L]
        V = self.vb[tab].transpose(0, 2, 1, 3).reshape(-1, self.H, 128)[:L]
        dt = self.dtype
        return decode_attention(storage_to_f64(self.q[i], dt), storage_to_f64(K, dt), storage_to_f64(V, dt),
                                1 / np.sqrt(128))

    def decode(self, P, chunk, split=False, noalloc=False, append=False):
        plan, info = decode_plan_shared(self.pool, self.seqs, self.Hq, P, chunk)
        q = to_device(self.q, self.dtype)
        out = torch.full((len(self.seqs), self.Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
        args = (torch.from_numpy(self.tables).cuda(), torch.from_numpy(self.lens).cuda(), 1 / np.sqrt(128),
                torch.from_numpy(plan).cuda(), info)
        k_new = v_new = None
        if append:
            # the newest token's rows, as the fused append stores them (same bits)
            rows = [(self.ora.table(s)[(self.ora.length(s) - 1) // BS], (self.ora.length(s) - 1) % BS)
                    for s in self.seqs]
            k_new = to_device(np.stack([self.kb[b, :, r, :] for b, r in rows]), self.dtype)
            v_new = to_device(np.stack([self.vb[b, :, r, :] for b, r in rows]), self.dtype)
        if noalloc:
            self.pool.paged_decode_noalloc(q, out, *args, k_new=k_new, v_new=v_new)
        else:
            ws = decode_workspace_bytes(info, self.Hq, 128)
            workspace = torch.zeros(max(ws // 4, 1), dtype=torch.float32, device="cuda")
            self.pool.paged_decode(q, out, *args, workspace, k_new=k_new, v_new=v_new, split=split)
        sync()
        return out.cpu().numpy().astype(np.float64), info

    def close(self):
        self.pool.close()
        del self.k_cache, self.v_cache
        torch.cuda.empty_cache()


CASES = [("f16", 4, 1), ("bf16", 4, 1), ("f16", 2, 4), ("bf16", 2, 8)]


@pytest.mark.parametrize("dtype,kv_heads,group", CASES, ids=lambda x: str(x))
def test_shared_decode_matches_oracle(dtype, kv_heads, group):
    case = ForkedCase(70 + group, dtype, kv_heads, group)
    try:
        ref = np.stack(oracle_map(case.oracle_out, range(len(case.seqs))))
        for P, chunk, kw in [(2048, 0, {}), (256, 64, {}), (512, 128, {"split": True}), (2048, 256, {"noalloc": True}),
                             (128, 0, {"append": True})]:
            print(f"\n[gpu] shared {dtype} H={kv_heads} G={group} P={P} chunk={chunk} {kw}", flush=True)
            out, info = case.decode(P, chunk, **kw)
            assert info.n_nodes > 0
            err = float(np.max(np.abs(out - ref)))
            print(f"[gpu]   nodes={info.n_nodes} items={info.n_shared_items} chunk_blocks={info.shared_chunk_blocks} "
                  f"partials={info.n_partials} max_err={err:.3e}", flush=True)
            assert np.isfinite(out).all() and err <= TOL[dtype], err
    finally:
        case.close()


@pytest.mark.parametrize("dtype,kv_heads,group", [("f16", 4, 1), ("f16", 2, 4), ("bf16", 2, 4)],
                         ids=lambda x: str(x))
def test_shared_decode_dominant_keys_outside_first_lane_group(dtype, kv_heads, group):
    """Every block's row 5 (lanes 16..31 of the score layout) dominates by
    about 43 in base 2 (see peaked_qk): the shared, narrow and own-block
    kernels must each take every row's maximum over all four lane groups, or
    the fp16 weights overflow.  Every output."""
    case = ForkedCase(90 + group, dtype, kv_heads, group, peaked=True)
    try:
        ref = np.stack(oracle_map(case.oracle_out, range(len(case.seqs))))
        for P, chunk in [(2048, 0), (256, 64)]:
            out, info = case.decode(P, chunk)
            assert info.n_nodes > 0
            err = float(np.max(np.abs(out - ref)))
            print(f"\n[gpu] peaked shared {dtype} H={kv_heads} G={group} P={P} chunk={chunk}: max err {err:.3e}",
                  flush=True)
            assert np.isfinite(out).all() and err <= TOL[dtype], err
    finally:
        case.close()



def test_shared_decode_replays_in_a_captured_graph():
    """The shared-block decode with its narrow launch on the library's side
    stream (forked from and joined back into the caller's stream by events),
    captured in a HIP graph after an eager call: each replay, with eager
    decodes between them, equals the eager output bit for bit."""
    case = ForkedCase(77, "f16", 4, 1, nan_fill=False)
    try:
        plan, info = decode_plan_shared(case.pool, case.seqs, case.Hq, 2048, 0)
        assert info.n_nodes > info.n_wide_nodes > 0  # wide and narrow launches both run
        q = to_device(case.q, "f16")
        args = (torch.from_numpy(case.tables).cuda(), torch.from_numpy(case.lens).cuda(), 1 / np.sqrt(128),
                torch.from_numpy(plan).cuda(), info)
        ws = decode_workspace_bytes(info, case.Hq, 128)
        workspace = torch.zeros(max(ws // 4, 1), dtype=torch.float32, device="cuda")
        shape = (len(case.seqs), case.Hq, 128)
        eager = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
        case.pool.paged_decode(q, eager, *args, workspace)  # creates the side stream
        sync()
        ref = eager.clone()
        err = float(np.max(np.abs(ref.cpu().numpy() - np.stack(oracle_map(case.oracle_out, range(len(case.seqs)))))))
        assert err <= TOL["f16"], err
        out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            case.pool.paged_decode(q, out, *args, workspace)
        for rep in range(3):
            out.fill_(float("nan"))
            g.replay()
            sync()
            assert torch.equal(out, ref), rep
            eager.fill_(float("nan"))
            case.pool.paged_decode(q, eager, *args, workspace)
            sync()
            assert torch.equal(eager, ref), rep
        print(f"\n[gpu] shared decode in a graph: 3 replays equal the eager call (oracle err {err:.2e})", flush=True)
    finally:
        case.close()
