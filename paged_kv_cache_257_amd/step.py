"""One decode iteration over a paged pool, as libpkv calls.

``step()`` is the production path: one call into the native stepper
(pkv_stepper_step) does the host half, the upload and the device half.
``prepare()`` + ``launch()`` spell the same iteration out call by call and
take options that switch fusions off, for comparisons.

Host (one C++ call, ``pkv_prepare_decode``): append the new token of every
sequence, take the copy-on-write pairs, build block tables, lengths and the
split-K plan into one pinned staging buffer.  One asynchronous copy uploads
it.  Device (HIP, in order on the compute stream): copy_blocks when there
are copy-on-write pairs, then one decode launch that also stores the new
tokens' K/V (``fused=False`` runs write_kv and the two-launch decode instead).

The upload runs on a side stream: the host prepares and uploads iteration
t+1 while the device still computes iteration t.  Three staging buffers
rotate; an event per buffer stops the host from rewriting a pinned buffer
still being copied, and another stops the copy from overwriting a device
buffer that kernels of an earlier iteration still read.
"""

from __future__ import annotations

import ctypes as C
from typing import Optional, Sequence

import numpy as np
import torch

from ._capi import BatchLayout, check, i32p
from .pool import Pool, _dptr, _stream_ptr

NBUF = 3
STEPPER_SLOTS = 8  # PKV_STEPPER_SLOTS in include/pkv.h
PARTITION_FILL = -1  # PKV_PARTITION_FILL in include/pkv.h


class DecodeIteration:
    def __init__(self, pool: Pool, max_batch: int, table_stride: int, num_q_heads: int,
                 partition_tokens: int = 0, append_tokens: int = 1, device: str = "cuda",
                 pipelined: bool = True):
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
        self.host = [torch.empty(self.nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(NBUF)]
        self.dev = [torch.empty(self.nbytes, dtype=torch.uint8, device=device) for _ in range(NBUF)]
        self.copy_done = [None] * NBUF
        self.compute_done = [None] * NBUF
        self.turn = 0
        self.copy_stream = torch.cuda.Stream(device=device) if pipelined else None
        ws = int(self.lib.pkv_decode_workspace_bound(max_batch, table_stride * bs, bs, partition_tokens,
                                                     num_q_heads, pool.desc.head_dim))
        if ws == 0:
            raise ValueError("bad decode geometry")
        # zeroed once: the decode's completion tickets start at zero and
        # every launch leaves them at zero
        self.workspace = torch.zeros(max(ws // 4, 1), dtype=torch.float32, device=device)
        # native stepper: its own staging slots
        self.slot_bytes = int(self.lib.pkv_stepper_slot_bytes(max_batch, table_stride, bs, partition_tokens))
        self.s_host = torch.empty(STEPPER_SLOTS * self.slot_bytes, dtype=torch.uint8, pin_memory=True)
        self.s_dev = torch.empty(STEPPER_SLOTS * self.slot_bytes, dtype=torch.uint8, device=device)
        h = C.c_void_p()
        check(self.lib, self.lib.pkv_stepper_create(
            pool.handle, max_batch, table_stride, num_q_heads, partition_tokens,
            self.s_host.data_ptr(), self.s_dev.data_ptr(), self.slot_bytes,
            self.workspace.data_ptr(), self.workspace.numel() * 4,
            self.copy_stream.cuda_stream if self.copy_stream is not None else None, C.byref(h)))
        self.stepper = h
        self._lay = BatchLayout()
        self._slot = C.c_int32()

    def close(self) -> None:
        if getattr(self, "stepper", None):
            self.lib.pkv_stepper_destroy(self.stepper)
            self.stepper = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 -- interpreter shutdown
            pass

    def step(self, seqs, q, out, k_new, v_new, scale: float, stream=None, events=None,
             host_meta: bool = False) -> BatchLayout:
        """One whole iteration in one native call.  ``seqs``: int32 numpy
        array (or sequence); ``events``: optional (start, stop) torch events
        attached to the decode dispatch (they time the kernel itself).  With ``host_meta`` the returned
        dict also holds host copies of the iteration's slots, pairs, tables
        and lengths."""
        seqs_np = seqs if isinstance(seqs, np.ndarray) and seqs.dtype == np.int32 else \
            np.ascontiguousarray(seqs, dtype=np.int32)
        e0 = e1 = None
        sp = _stream_ptr(stream)
        if events is not None:
            for e in events:
                if not e.cuda_event:  # torch creates the HIP event on first record
                    e.record(torch.cuda.current_stream() if stream is None else stream)
            e0, e1 = events[0].cuda_event, events[1].cuda_event
        check(self.lib, self.lib.pkv_stepper_step(
            self.stepper, seqs_np.ctypes.data_as(C.POINTER(C.c_int32)), len(seqs_np), q.data_ptr(),
            k_new.data_ptr(), v_new.data_ptr(), out.data_ptr(), float(scale), sp, e0, e1,
            C.byref(self._lay), C.byref(self._slot)))
        if not host_meta:
            return self._lay
        lay, n = self._lay, len(seqs_np)
        hv = self.s_host.numpy()[self._slot.value * self.slot_bytes:(self._slot.value + 1) * self.slot_bytes]
        return dict(
            layout=lay, info=lay.plan, n=n, npairs=lay.n_pairs,
            host_slots=hv[lay.off_slots:lay.off_slots + 8 * n].view(np.int64).copy(),
            host_pairs=hv[lay.off_pairs:lay.off_pairs + 8 * lay.n_pairs].view(np.int32).reshape(-1, 2).copy(),
            host_tables=hv[lay.off_tables:lay.off_tables + 4 * n * self.stride].view(np.int32)
            .reshape(n, self.stride).copy(),
            host_lens=hv[lay.off_lens:lay.off_lens + 4 * n].view(np.int32).copy())

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
        self.turn = (k + 1) % NBUF
        if self.copy_done[k] is not None:
            self.copy_done[k].synchronize()
        host, dev = self.host[k], self.dev[k]
        lay = BatchLayout()
        a = self.append_tokens if append else 0
        if self.P == PARTITION_FILL:
            raise ValueError("fill-mode partitioning is chosen by the native stepper (step()); "
                             "prepare() takes a concrete partition size or 0")
        check(self.lib, self.lib.pkv_prepare_decode(self.pool.handle, i32p(seqs_np), n, a, self.stride,
                                                    self.P, self.Hq, host.data_ptr(), self.nbytes,
                                                    C.byref(lay)))
        compute = torch.cuda.current_stream() if stream is None else stream
        cs = self.copy_stream if self.copy_stream is not None else compute
        if self.copy_stream is not None and self.compute_done[k] is not None:
            cs.wait_event(self.compute_done[k])
        with torch.cuda.stream(cs):
            dev[:lay.bytes].copy_(host[:lay.bytes], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(cs)
        self.copy_done[k] = ev
        hv = host.numpy()
        return dict(
            buf=k, layout=lay, info=lay.plan, n=n, npairs=lay.n_pairs,
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
               events: Optional[tuple] = None, fused: bool = True, fused_append: bool = True) -> None:
        """Device half.  ``fused``: one decode launch with the split-K combine
        inside (else partition kernel + combine kernel).  ``fused_append``: the
        decode stores the new tokens' K/V (else write_kv does).  ``events`` =
        (before, after) torch events recorded around the decode partition
        kernel (for timing it alone)."""
        pool, lib = self.pool, self.lib
        s = torch.cuda.current_stream() if stream is None else stream
        if self.copy_stream is not None:
            s.wait_event(self.copy_done[meta["buf"]])
        sp = _stream_ptr(s)
        if meta["npairs"]:
            pool.copy_blocks(meta["pairs"], s)
        if k_new is not None and not fused_append:
            pool.write_kv(k_new, v_new, meta["slots"], s)
        kn, vn = (k_new, v_new) if fused_append else (None, None)
        info = meta["info"]
        ws_bytes = self.workspace.numel() * 4
        args = (pool.handle, _dptr(q), _dptr(kn), _dptr(vn), _dptr(out), meta["n"], self.Hq,
                _dptr(meta["tables"]), self.stride, _dptr(meta["lens"]), float(scale),
                _dptr(meta["plan"]), C.byref(info), _dptr(self.workspace), ws_bytes, sp)
        if events is not None:
            events[0].record(s)
        if fused:
            check(lib, lib.pkv_paged_decode(*args))
        else:
            check(lib, lib.pkv_paged_decode_partitions(*args))
        if events is not None:
            events[1].record(s)
        if not fused:
            check(lib, lib.pkv_paged_decode_reduce(*args))
        ev = torch.cuda.Event()
        ev.record(s)
        self.compute_done[meta["buf"]] = ev
