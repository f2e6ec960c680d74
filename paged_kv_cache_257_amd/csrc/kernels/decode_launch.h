// Decode entry points shared inside the library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "../host/pool_internal.h"

#define PKV_DECODE_ARGS                                                                          \
  const pkv_pool *pool, const void *q, const void *k_new, const void *v_new, float *out,        \
      int32_t num_seqs, int32_t num_q_heads, const int32_t *block_tables, int32_t table_stride, \
      const int32_t *context_lens, float scale, const int32_t *plan,                            \
      const pkv_decode_plan_info *info, void *workspace, size_t workspace_bytes, void *stream

namespace pkv {

// pkv_paged_decode with optional start / stop events attached to the decode
// dispatch (either may be null; both null is a plain launch).
pkv_status paged_decode_timed(PKV_DECODE_ARGS, hipEvent_t ev_start, hipEvent_t ev_stop);

}  // namespace pkv
