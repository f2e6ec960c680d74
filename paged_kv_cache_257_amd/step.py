"""One decode iteration over a paged pool, as libpkv calls.

Host (one C++ call, ``pkv_prepare_decode``): append the new token of every
sequence, take the copy-on-write pairs, build block tables, lengths and the
split-K plan into one pinned staging buffer.  One asynchronous copy uploads
it.  Device (HIP kernels, same stream, in order): copy_blocks, write_kv,
the decode partition kernel, the split-K reduce.

Two staging buffers alternate; an event per buffer keeps the host from
overwriting one whose upload may still be in flight.
"""

from __future__ import annotations

import ctypes as C
from typing import Optional, Sequence

import numpy as np
import torch

from ._capi import BatchLayout, PlanInfo, check, i32p
from .pool import Pool, _dptr, _stream_ptr, decode_workspace_bytes


class DecodeIteration:
    def __init__(self, pool: Pool, max_batch: int, table_stride: int, num_q_heads: int,
                 partition_tokens: int = 0, append_tokens: int = 1, device: str = "cuda"):
        self.pool = pool
        self.lib = pool.lib
        self.B = max_batch
        self.stride = table_stride
        self.Hq = num_q_heads
        self.P = partition_tokens
        self.append_tokens = append_tokens
        bs = pool.desc.block_size
        self.nbytes = int(self.lib.pkv_prepare_decode_bytes(max_batch, append_tokens, table_stride,
                                                            bs, partition_tokens))
        if self.nbytes == 0:
            raise ValueError("bad staging geometry")
        self.host = [torch.empty(self.nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
        self.dev = [torch.empty(self.nbytes, dtype=torch.uint8, device=device) for _ in range(2)]
        self.events = [None, None]
        self.turn = 0
        P_eff = partition_tokens or 512
        max_parts = -(-table_stride * bs // P_eff)
        worst = PlanInfo(max_batch, bs, P_eff, 0, 0, max_batch * max_parts, 0, 0)
        ws = decode_workspace_bytes(worst, num_q_heads, pool.desc.head_dim)
        self.workspace = torch.empty(max(ws // 4, 1), dtype=torch.float32, device=device)

    @staticmethod
    def _view(buf: torch.Tensor, off: int, count: int, dtype, shape=None):
        nbytes = count * torch.empty(0, dtype=dtype).element_size()
        t = buf[off:off + nbytes].view(dtype)
        return t if shape is None else t.view(*shape)

    def prepare(self, seqs: Sequence[int], append: bool = True, stream=None) -> dict:
        """Host half of the iteration; returns the metadata's device views."""
        seqs_np = np.ascontiguousarray(seqs, dtype=np.int32)
        n = len(seqs_np)
        if n > self.B:
            raise ValueError("batch larger than max_batch")
        k = self.turn
        self.turn ^= 1
        if self.events[k] is not None:
            self.events[k].synchronize()
        host, dev = self.host[k], self.dev[k]
        lay = BatchLayout()
        a = self.append_tokens if append else 0
        check(self.lib, self.lib.pkv_prepare_decode(self.pool.handle, i32p(seqs_np), n, a, self.stride,
                                                    self.P, host.data_ptr(), self.nbytes, C.byref(lay)))
        s = torch.cuda.current_stream() if stream is None else stream
        with torch.cuda.stream(s):
            dev[:lay.bytes].copy_(host[:lay.bytes], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(s)
        self.events[k] = ev
        hv = host.numpy()
        return dict(
            layout=lay, info=lay.plan, n=n, npairs=lay.n_pairs,
            slots=self._view(dev, lay.off_slots, n * a, torch.int64),
            pairs=self._view(dev, lay.off_pairs, 2 * lay.n_pairs, torch.int32, (lay.n_pairs, 2)),
            tables=self._view(dev, lay.off_tables, n * self.stride, torch.int32, (n, self.stride)),
            lens=self._view(dev, lay.off_lens, n, torch.int32),
            plan=self._view(dev, lay.off_plan, max(lay.plan.plan_ints, 1), torch.int32),
            host_slots=hv[lay.off_slots:lay.off_slots + 8 * n * a].view(np.int64).copy(),
            host_pairs=hv[lay.off_pairs:lay.off_pairs + 8 * lay.n_pairs].view(np.int32).reshape(-1, 2).copy(),
            host_tables=hv[lay.off_tables:lay.off_tables + 4 * n * self.stride].view(np.int32)
            .reshape(n, self.stride).copy(),
            host_lens=hv[lay.off_lens:lay.off_lens + 4 * n].view(np.int32).copy(),
        )

    def launch(self, meta: dict, q, out, k_new=None, v_new=None, scale: float = 1.0, stream=None,
               events: Optional[tuple] = None) -> None:
        """Device half.  ``events`` = (before, after) torch events recorded
        around the decode partition kernel (for timing it alone)."""
        pool, lib = self.pool, self.lib
        sp = _stream_ptr(stream)
        if meta["npairs"]:
            pool.copy_blocks(meta["pairs"], stream)
        if k_new is not None:
            pool.write_kv(k_new, v_new, meta["slots"], stream)
        info = meta["info"]
        ws_bytes = self.workspace.numel() * 4
        args = (pool.handle, _dptr(q), _dptr(out), meta["n"], self.Hq, _dptr(meta["tables"]),
                self.stride, _dptr(meta["lens"]), float(scale), _dptr(meta["plan"]), C.byref(info),
                _dptr(self.workspace), ws_bytes, sp)
        s = torch.cuda.current_stream() if stream is None else stream
        if events is not None:
            events[0].record(s)
        check(lib, lib.pkv_paged_decode_partitions(*args))
        if events is not None:
            events[1].record(s)
        check(lib, lib.pkv_paged_decode_reduce(*args))
