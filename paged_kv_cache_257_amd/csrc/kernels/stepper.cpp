// Decode-iteration stepper: the host half (pkv_prepare_decode) and the device
// half (upload, copy-on-write copies, one decode launch) of a continuous-
// batching iteration ("PagedAttention e continuous batching", 01 · Conceito,
// paragraph 7: running sequences advance one token per iteration) in one
// native call, so that a caller pays one foreign-function call per iteration.
//
// The metadata of iteration t is uploaded on a separate copy stream while the
// compute stream still runs earlier iterations, and the compute stream never
// waits on another stream: the host does the waiting.  Eight staging slots
// rotate in two groups of four.  Before reusing a slot the host waits for the
// completion event of its group from the previous round (recorded after the
// group's last launch, four to eight iterations back, normally long finished);
// after queuing the upload it waits for the copy (a few microseconds of DMA)
// and only then launches.  That wait synchronises the copy stream, which
// waits on the copy itself.  A host wait on an event recorded behind the copy
// was measured to return only after the decodes already queued on the compute
// stream had finished (HIP maps many streams onto a few hardware queues, and
// the two can share one), leaving the GPU idle until the host caught up: with
// eight steppers in rotation, a 30 us gap every eighth iteration.
// An event record on the compute stream costs GPU time, so one is recorded
// per group, not per launch.  The library creates only these events; every
// buffer is the caller's.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>
#include <vector>

#include "../host/pool_internal.h"
#include "decode_launch.h"

using pkv::fail;

namespace {
constexpr int kSlots = 8;
constexpr int kGroup = 4;  // slots per completion event
}

struct pkv_stepper {
  pkv_pool* pool = nullptr;
  int32_t max_seqs = 0, stride = 0, num_q_heads = 0, partition_tokens = 0;
  char* host = nullptr;
  char* dev = nullptr;
  size_t slot_bytes = 0;
  void* workspace = nullptr;
  size_t workspace_bytes = 0;
  hipStream_t copy = nullptr;
  hipEvent_t compute_done[kSlots / kGroup] = {};
  bool used[kSlots] = {};
  int next = 0;
  hipStream_t last_stream = nullptr;  // compute stream of the latest launch
  bool pending = false;               // launches since the last group event
  // fill mode (partition_tokens == PKV_PARTITION_FILL): the decode's
  // workgroups per work item and resident workgroups, and length scratch
  int32_t fill_wpi = 0;
  int64_t fill_resident = 0;
  std::vector<int32_t> fill_lens;
};

namespace {

pkv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

extern "C" {

size_t pkv_stepper_slot_bytes(int32_t max_seqs, int32_t table_stride, int32_t block_size,
                              int32_t partition_tokens) {
  const size_t b = pkv_prepare_decode_bytes(max_seqs, 1, table_stride, block_size, partition_tokens);
  return (b + 255) / 256 * 256;
}

pkv_status pkv_stepper_create(pkv_pool* pool, int32_t max_seqs, int32_t table_stride,
                              int32_t num_q_heads, int32_t partition_tokens, void* staging_host,
                              void* staging_dev, size_t slot_bytes, void* workspace,
                              size_t workspace_bytes, void* copy_stream, pkv_stepper** out) {
  if (!pool || !out || !staging_host || !staging_dev)
    return fail(PKV_E_BAD_ARG, "null pool, staging buffer or out");
  if (max_seqs < 1 || table_stride < 1 || num_q_heads < 1)
    return fail(PKV_E_BAD_ARG, "bad stepper geometry");
  const size_t need = pkv_stepper_slot_bytes(max_seqs, table_stride, pool->desc.block_size,
                                             partition_tokens);
  if (need == 0 || slot_bytes < need)
    return fail(PKV_E_BAD_ARG, "staging slot too small: need " + std::to_string(need) + " bytes");
  if (slot_bytes % 256 != 0) return fail(PKV_E_BAD_ARG, "slot_bytes must be a multiple of 256");
  int32_t wpi = 0;
  int64_t resident = 0;
  if (partition_tokens == PKV_PARTITION_FILL) {
    if (pkv_status st = pkv_decode_occupancy(pool, num_q_heads, &wpi, &resident)) return st;
  }
  pkv_stepper* s = new pkv_stepper();
  s->pool = pool;
  s->fill_wpi = wpi;
  s->fill_resident = resident;
  s->max_seqs = max_seqs;
  s->stride = table_stride;
  s->num_q_heads = num_q_heads;
  s->partition_tokens = partition_tokens;
  s->host = static_cast<char*>(staging_host);
  s->dev = static_cast<char*>(staging_dev);
  s->slot_bytes = slot_bytes;
  s->workspace = workspace;
  s->workspace_bytes = workspace_bytes;
  s->copy = static_cast<hipStream_t>(copy_stream);
  for (int g = 0; g < kSlots / kGroup; ++g) {
    pkv_status st = hip_status(hipEventCreateWithFlags(&s->compute_done[g], hipEventDisableTiming),
                               "hipEventCreateWithFlags");
    if (st != PKV_OK) {
      pkv_stepper_destroy(s);
      return st;
    }
  }
  *out = s;
  return PKV_OK;
}

pkv_status pkv_stepper_destroy(pkv_stepper* s) {
  if (!s) return PKV_OK;
  if (s->pending && s->last_stream) {
    // launches after the last group event: record one more and wait for it
    if (hipEventRecord(s->compute_done[0], s->last_stream) == hipSuccess)
      (void)hipEventSynchronize(s->compute_done[0]);
  }
  for (int g = 0; g < kSlots / kGroup; ++g)
    if (s->compute_done[g]) {
      (void)hipEventSynchronize(s->compute_done[g]);
      (void)hipEventDestroy(s->compute_done[g]);
    }
  delete s;
  return PKV_OK;
}

pkv_status pkv_stepper_step(pkv_stepper* s, const int32_t* seqs, int32_t n_seqs, const void* q,
                            const void* k_new, const void* v_new, float* out, float scale,
                            void* stream, void* ev_before, void* ev_after,
                            pkv_batch_layout* layout_out, int32_t* slot_out) {
  if (!s) return fail(PKV_E_BAD_ARG, "null stepper");
  if (n_seqs > s->max_seqs) return fail(PKV_E_BAD_ARG, "batch larger than the stepper's max_seqs");
  hipStream_t cs = static_cast<hipStream_t>(stream);
  hipStream_t up = s->copy ? s->copy : cs;
  const int k = s->next;
  char* host = s->host + size_t(k) * s->slot_bytes;
  char* dev = s->dev + size_t(k) * s->slot_bytes;
  if (s->used[k]) {  // the iterations that last used this slot's group have finished
    if (pkv_status st = hip_status(hipEventSynchronize(s->compute_done[k / kGroup]), "hipEventSynchronize"))
      return st;
  }
  int32_t P = s->partition_tokens;
  if (P == PKV_PARTITION_FILL) {
    // the batch's lengths after this iteration's append
    s->fill_lens.resize(size_t(std::max(n_seqs, 0)));
    for (int32_t i = 0; i < n_seqs; ++i) {
      if (pkv_status st = pkv_seq_length(s->pool, seqs[i], &s->fill_lens[i])) return st;
      s->fill_lens[i] += 1;
    }
    P = pkv_decode_fill_partition(s->fill_lens.data(), n_seqs, s->pool->desc.block_size, s->fill_wpi,
                                  s->fill_resident, PKV_FILL_MIN_TOKENS);
    if (P == 0) P = pkv::kDefaultPartitionTokens;
  }
  pkv_batch_layout lay{};
  if (pkv_status st = pkv_prepare_decode(s->pool, seqs, n_seqs, 1, s->stride, P, s->num_q_heads, host,
                                                 s->slot_bytes, &lay))
    return st;  // the pool is unchanged
  s->next = (k + 1) % kSlots;
  if (layout_out) *layout_out = lay;
  if (slot_out) *slot_out = k;
  if (pkv_status st = hip_status(hipMemcpyAsync(dev, host, size_t(lay.bytes), hipMemcpyHostToDevice, up),
                                 "hipMemcpyAsync"))
    return st;
  if (s->copy) {
    if (pkv_status st = hip_status(hipStreamSynchronize(up), "hipStreamSynchronize")) return st;
  }
  if (lay.n_pairs > 0) {
    if (pkv_status st = pkv_copy_blocks(s->pool, reinterpret_cast<const int32_t*>(dev + lay.off_pairs),
                                        lay.n_pairs, cs))
      return st;
  }
  if (pkv_status st = pkv::paged_decode_timed(
          s->pool, q, k_new, v_new, out, n_seqs, s->num_q_heads,
          reinterpret_cast<const int32_t*>(dev + lay.off_tables), s->stride,
          reinterpret_cast<const int32_t*>(dev + lay.off_lens), scale,
          reinterpret_cast<const int32_t*>(dev + lay.off_plan), &lay.plan, s->workspace,
          s->workspace_bytes, cs, static_cast<hipEvent_t>(ev_before), static_cast<hipEvent_t>(ev_after)))
    return st;
  s->used[k] = true;
  s->last_stream = cs;
  s->pending = true;
  if (k % kGroup != kGroup - 1) return PKV_OK;
  s->pending = false;
  return hip_status(hipEventRecord(s->compute_done[k / kGroup], cs), "hipEventRecord");
}

}  // extern "C"
