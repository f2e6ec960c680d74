// Split-K work plan for paged decode (host, CPU only).
//
// A sequence of L tokens is cut into partitions of P tokens; each
// (sequence, partition) is one work item.  Long partitions go first: the GPU
// dispatches workgroups in grid order to whichever compute unit frees up, so
// a longest-first list behaves like greedy longest-processing-time
// scheduling and leaves short items to fill the tail of the launch.
#include <algorithm>
#include <vector>

#include "pool_internal.h"

using pkv::fail;

namespace {

constexpr int32_t kDefaultPartitionTokens = 512;

pkv_status check_lens(const int32_t* lens, int32_t n, int32_t bs, int32_t& P, int32_t& max_len) {
  if (n < 0 || (n > 0 && !lens)) return fail(PKV_E_BAD_ARG, "bad context_lens");
  if (bs < 1) return fail(PKV_E_BAD_ARG, "bad block_size");
  if (P == 0) P = kDefaultPartitionTokens;
  if (P < bs || P % bs != 0)
    return fail(PKV_E_BAD_ARG, "partition_tokens must be a positive multiple of block_size");
  max_len = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (lens[i] < 1) return fail(PKV_E_BAD_ARG, "every context length must be >= 1");
    max_len = std::max(max_len, lens[i]);
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_decode_plan_ints(const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                                int32_t partition_tokens, int32_t* plan_ints) {
  if (!plan_ints) return fail(PKV_E_BAD_ARG, "null plan_ints");
  int32_t P = partition_tokens, max_len = 0;
  if (pkv_status st = check_lens(context_lens, num_seqs, block_size, P, max_len)) return st;
  int64_t work = 0, reduce = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    int64_t parts = (int64_t(context_lens[i]) + P - 1) / P;
    work += parts;
    reduce += parts > 1;
  }
  int64_t total = 2 * work + num_seqs + reduce;
  if (total > INT32_MAX) return fail(PKV_E_BAD_ARG, "plan too large");
  *plan_ints = int32_t(total);
  return PKV_OK;
}

pkv_status pkv_decode_plan(const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                           int32_t partition_tokens, int32_t* plan, int32_t cap,
                           pkv_decode_plan_info* info) {
  if (!info) return fail(PKV_E_BAD_ARG, "null info");
  int32_t need = 0;
  if (pkv_status st = pkv_decode_plan_ints(context_lens, num_seqs, block_size, partition_tokens, &need))
    return st;
  if (cap < need || (need > 0 && !plan)) return fail(PKV_E_BAD_ARG, "plan buffer too small");
  int32_t P = partition_tokens, max_len = 0;
  check_lens(context_lens, num_seqs, block_size, P, max_len);
  const int32_t pblocks = P / block_size;

  // work items bucketed by their block count (counting sort, longest first,
  // ties in (sequence, partition) order)
  std::vector<std::vector<std::pair<int32_t, int32_t>>> by_len(pblocks + 1);
  int32_t n_work = 0, n_reduce = 0, n_partials = 0;
  int32_t* part_offset = plan;  // filled after the work list is laid out
  std::vector<int32_t> offsets(num_seqs, -1), reduce;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t L = context_lens[i];
    const int32_t nblk = (L + block_size - 1) / block_size;
    const int32_t parts = (L + P - 1) / P;
    for (int32_t p = 0; p < parts; ++p) {
      int32_t blocks = std::min(pblocks, nblk - p * pblocks);
      by_len[blocks].emplace_back(i, p);
    }
    n_work += parts;
    if (parts > 1) {
      offsets[i] = n_partials;
      n_partials += parts;
      reduce.push_back(i);
      n_reduce++;
    }
  }
  int32_t w = 0;
  for (int32_t b = pblocks; b >= 1; --b)
    for (const auto& it : by_len[b]) {
      plan[2 * w] = it.first;
      plan[2 * w + 1] = it.second;
      w++;
    }
  part_offset = plan + 2 * n_work;
  std::copy(offsets.begin(), offsets.end(), part_offset);
  std::copy(reduce.begin(), reduce.end(), part_offset + num_seqs);

  info->num_seqs = num_seqs;
  info->block_size = block_size;
  info->partition_tokens = P;
  info->n_work = n_work;
  info->n_reduce = n_reduce;
  info->n_partials = n_partials;
  info->plan_ints = need;
  info->max_context_len = max_len;
  return PKV_OK;
}

size_t pkv_decode_workspace_bytes(const pkv_decode_plan_info* info, int32_t num_q_heads,
                                  int32_t head_dim) {
  if (!info || num_q_heads < 1 || head_dim < 1) return 0;
  // partial o (head_dim floats) + (m, l) per (partial, query head)
  return size_t(info->n_partials) * size_t(num_q_heads) * (size_t(head_dim) + 2) * sizeof(float);
}

}  // extern "C"
