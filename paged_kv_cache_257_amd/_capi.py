"""ctypes declarations of the libpkv C ABI (include/pkv.h).

Argument marshalling only.  ``load()`` opens the in-tree library and raises
if it has not been built: there is no fallback path.
"""

from __future__ import annotations

import ctypes as C
import os

LIBDIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib")

OK, E_NO_BLOCKS, E_BAD_SEQ, E_BAD_ARG, E_TABLE_FULL, E_HIP, E_UNSUPPORTED, E_NO_SLOTS = range(8)
STATUS_KIND = {E_NO_BLOCKS: "no_blocks", E_BAD_SEQ: "bad_seq", E_BAD_ARG: "bad_arg",
               E_TABLE_FULL: "table_full", E_HIP: "hip", E_UNSUPPORTED: "unsupported",
               E_NO_SLOTS: "no_slots"}
DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
NOALLOC_SCRATCH_BYTES = 32 << 20  # PKV_NOALLOC_SCRATCH_BYTES of include/pkv.h
MAX_SHARED_RECORDS = 16           # PKV_MAX_SHARED_RECORDS of include/pkv.h
PROBE_MODES = {"regs": 0, "cached": 1, "lds": 2}  # PKV_PROBE_* of include/pkv.h


class PoolDesc(C.Structure):
    _fields_ = [("num_blocks", C.c_int32), ("block_size", C.c_int32),
                ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("max_blocks_per_seq", C.c_int32), ("dtype", C.c_int32)]


class Stats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("free_blocks", "used_blocks", "alloc_failures",
                                         "tail_waste_slots", "shared_blocks", "cow_copies",
                                         "forks", "live_seqs")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class PlanInfo(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("num_seqs", "block_size", "partition_tokens", "n_work",
                                         "n_reduce", "n_partials", "plan_ints", "max_context_len",
                                         "shared_kv", "n_nodes", "n_wide_nodes", "n_shared_items",
                                         "n_narrow_items", "shared_chunk_blocks", "narrow_chunk_blocks",
                                         "shared_group", "off_shared", "item_blocks")]


class PrefillPlanInfo(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("num_seqs", "num_q_heads", "num_kv_heads", "tile_tokens",
                                         "n_work", "total_q", "max_context_len", "plan_ints",
                                         "n_split", "n_partials")]


class Utilisation(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("requests", "tokens_used", "naive_reserved_tokens",
                                         "paged_blocks", "paged_reserved_tokens",
                                         "naive_waste_tokens", "paged_waste_tokens")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class HybridStats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("free_slots", "used_slots", "refusals", "state_copies")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class Request(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("arrival", "prompt_len", "output_len", "klass", "prefix_id",
                                         "prefix_len")]


class SchedConfig(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("max_batch_tokens", "chunk_tokens", "max_running")]


class SchedItem(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("request", "seq", "kind", "pos", "n_tokens")]


class SchedStepInfo(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("iteration", "n_items", "prefill_tokens", "decode_tokens",
                                         "admitted", "preempted", "finished", "rejected")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class RequestState(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("state", "seq", "admitted_at", "first_token_at", "finished_at",
                                         "generated", "preemptions", "prefix_hit_tokens")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class SchedStats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("iterations", "waiting", "running", "finished", "rejected",
                                         "preemptions", "prompt_tokens_admitted", "prefix_hit_tokens",
                                         "prefill_tokens", "decode_tokens")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class BatchLayout(C.Structure):
    _fields_ = [("n_seqs", C.c_int32), ("append_tokens", C.c_int32), ("n_pairs", C.c_int32),
                ("table_stride", C.c_int32), ("off_slots", C.c_int64), ("off_pairs", C.c_int64),
                ("off_tables", C.c_int64), ("off_lens", C.c_int64), ("off_plan", C.c_int64),
                ("bytes", C.c_int64), ("plan", PlanInfo)]


class PkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libpkv: {STATUS_KIND.get(status, status)}: {msg}")
        self.status = status
        self.kind = STATUS_KIND.get(status, str(status))


P = C.c_void_p
I32 = C.c_int32
PI32 = C.POINTER(C.c_int32)
PI64 = C.POINTER(C.c_int64)

# pool, q, k_new, v_new, out, num_seqs, num_q_heads, tables, stride, lens, scale,
# plan, info, workspace, workspace_bytes, stream
DECODE_ARGS = [P, P, P, P, P, I32, I32, P, I32, P, C.c_float, P, C.POINTER(PlanInfo), P,
               C.c_size_t, P]

# name -> (argtypes); every function returns pkv_status (int) unless listed
SIGNATURES = {
    "pkv_pool_create": [C.POINTER(PoolDesc), P, P, PI32, C.POINTER(P)],
    "pkv_pool_destroy": [P],
    "pkv_pool_reset": [P],
    "pkv_pool_get_desc": [P, C.POINTER(PoolDesc)],
    "pkv_seq_alloc": [P, I32, PI32, PI64],
    "pkv_seq_append": [P, I32, I32, PI64],
    "pkv_seq_append_batch": [P, PI32, I32, I32, PI64],
    "pkv_seq_fork": [P, I32, PI32],
    "pkv_seq_fork_prefix": [P, I32, I32, PI32],
    "pkv_sched_create": [P, C.POINTER(SchedConfig), C.POINTER(Request), I32, C.POINTER(P)],
    "pkv_sched_destroy": [P],
    "pkv_sched_step": [P, C.POINTER(SchedItem), I32, C.POINTER(SchedStepInfo)],
    "pkv_sched_request": [P, I32, C.POINTER(RequestState)],
    "pkv_sched_stats": [P, C.POINTER(SchedStats)],
    "pkv_seq_free": [P, I32],
    "pkv_seq_free_batch": [P, PI32, I32],
    "pkv_seq_fork_batch": [P, PI32, I32, PI32],
    "pkv_seq_length": [P, I32, PI32],
    "pkv_seq_table": [P, I32, PI32, I32, PI32],
    "pkv_seq_slots": [P, I32, I32, I32, PI64],
    "pkv_live_seqs": [P, PI32, I32, PI32],
    "pkv_free_list": [P, PI32, I32, PI32],
    "pkv_refcounts": [P, PI32],
    "pkv_stats": [P, C.POINTER(Stats)],
    "pkv_take_cow": [P, PI32, I32, PI32],
    "pkv_build_batch": [P, PI32, I32, PI32, I32, PI32],
    "pkv_utilisation": [PI32, I32, I32, I32, C.POINTER(Utilisation)],
    "pkv_hybrid_create": [P, I32, C.c_int64, P, PI32, C.POINTER(P)],
    "pkv_hybrid_destroy": [P],
    "pkv_hybrid_admit": [P, I32, PI32, PI32, PI64],
    "pkv_hybrid_fork": [P, I32, PI32, PI32],
    "pkv_hybrid_free": [P, I32],
    "pkv_hybrid_slot": [P, I32, PI32],
    "pkv_hybrid_take_copies": [P, PI32, I32, PI32],
    "pkv_hybrid_stats": [P, C.POINTER(HybridStats)],
    "pkv_hybrid_copy_states": [P, P, I32, P],
    "pkv_hybrid_plan": [C.c_int64, C.c_int64, I32, C.c_int64, C.c_int64, PI32, PI32, PI32],
    "pkv_decode_plan_ints": [PI32, I32, I32, I32, PI32],
    "pkv_decode_plan": [PI32, I32, I32, I32, PI32, I32, C.POINTER(PlanInfo)],
    "pkv_decode_plan_shared_ints": [P, PI32, I32, I32, PI32],
    "pkv_decode_plan_shared": [P, PI32, I32, I32, I32, I32, PI32, I32, C.POINTER(PlanInfo)],
    "pkv_decode_workspace_bytes": [C.POINTER(PlanInfo), I32, I32],
    "pkv_decode_workspace_bound": [I32, I32, I32, I32, I32, I32],
    "pkv_default_partition_tokens": [],
    "pkv_decode_fill_partition": [PI32, I32, I32, I32, C.c_int64, I32],
    "pkv_decode_occupancy": [P, I32, PI32, PI64],
    "pkv_prefill_plan_ints": [PI32, PI32, I32, I32, I32, I32, PI32],
    "pkv_prefill_plan": [PI32, PI32, I32, I32, I32, I32, PI32, I32, C.POINTER(PrefillPlanInfo)],
    "pkv_prefill_workspace_bytes": [C.POINTER(PrefillPlanInfo), I32],
    "pkv_prepare_decode_bytes": [I32, I32, I32, I32, I32],
    "pkv_prepare_decode": [P, PI32, I32, I32, I32, I32, I32, P, C.c_size_t, C.POINTER(BatchLayout)],
    "pkv_batch_shared_kv": [P, PI32, I32, PI32],
    "pkv_stepper_slot_bytes": [I32, I32, I32, I32],
    "pkv_stepper_create": [P, I32, I32, I32, I32, P, P, C.c_size_t, P, C.c_size_t, P, C.POINTER(P)],
    "pkv_stepper_destroy": [P],
    "pkv_stepper_step": [P, PI32, I32, P, P, P, P, C.c_float, P, P, P, C.POINTER(BatchLayout),
                         PI32],
    "pkv_copy_blocks": [P, P, I32, P],
    "pkv_write_kv": [P, P, P, P, I32, P],
    "pkv_read_kv": [P, P, I32, P, P, P],
    "pkv_paged_decode": DECODE_ARGS,
    "pkv_paged_decode_partitions": DECODE_ARGS,
    "pkv_paged_decode_reduce": DECODE_ARGS,
    "pkv_paged_decode_noalloc": [P, P, P, P, P, I32, I32, P, I32, P, C.c_float, P, C.POINTER(PlanInfo), P],
    "pkv_paged_prefill": [P, P, P, I32, I32, P, I32, P, C.c_float, P, C.POINTER(PrefillPlanInfo), P,
                          C.c_size_t, P],
    "pkv_gather_probe": [P, P, I32, P, I32, P, C.POINTER(PlanInfo), I32, I32, I32, P, P],
    "pkv_last_error": [],
}
RESTYPES = {"pkv_last_error": C.c_char_p, "pkv_decode_workspace_bytes": C.c_size_t,
            "pkv_decode_workspace_bound": C.c_size_t, "pkv_default_partition_tokens": C.c_int32,
            "pkv_decode_fill_partition": C.c_int32,
            "pkv_prefill_workspace_bytes": C.c_size_t,
            "pkv_prepare_decode_bytes": C.c_size_t, "pkv_stepper_slot_bytes": C.c_size_t}
DEVICE_FUNCS = ("pkv_copy_blocks", "pkv_write_kv", "pkv_read_kv", "pkv_paged_decode", "pkv_paged_decode_partitions",
                "pkv_decode_occupancy",
                "pkv_paged_decode_reduce", "pkv_paged_decode_noalloc", "pkv_paged_prefill", "pkv_hybrid_copy_states", "pkv_gather_probe",
                "pkv_stepper_slot_bytes", "pkv_stepper_create",
                "pkv_stepper_destroy", "pkv_stepper_step")

_LIBS = {}


def lib_path(host_only: bool = False) -> str:
    return os.path.join(LIBDIR, "libpkv_host.so" if host_only else "libpkv.so")


def load(host_only: bool = False):
    """Open libpkv.so (or the host-only allocator library) and declare it."""
    key = bool(host_only)
    if key in _LIBS:
        return _LIBS[key]
    path = lib_path(host_only)
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python __graft_entry__.py build` "
                          "(or paged_kv_cache_257_amd.build.build()) first")
    lib = C.CDLL(path)
    for name, args in SIGNATURES.items():
        if host_only and name in DEVICE_FUNCS:
            continue
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = RESTYPES.get(name, C.c_int)
    _LIBS[key] = lib
    return lib


def check(lib, status: int) -> None:
    if status != OK:
        raise PkvError(status, lib.pkv_last_error().decode())


def i32p(arr):
    """int32 numpy array -> ctypes pointer (None for None)."""
    return None if arr is None else arr.ctypes.data_as(PI32)


def i64p(arr):
    return None if arr is None else arr.ctypes.data_as(PI64)
