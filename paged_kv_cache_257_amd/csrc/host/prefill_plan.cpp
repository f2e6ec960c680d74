// Host work list of a chunked-prefill launch (pkv_prefill_plan).
//
// The lesson's scheduler slices long prefills into chunks ("PagedAttention
// e continuous batching", 01 · Conceito, the scheduler paragraph); a launch
// takes one chunk of each of several sequences.  Work items are tiles of
// consecutive query tokens; a tile's cost is the number of keys its last
// token attends, so items are sorted by that, largest first, and the
// in-order workgroup dispatcher fills the tail of the launch with the
// cheap ones.
#include <algorithm>
#include <numeric>
#include <vector>

#include "pool_internal.h"

using pkv::fail;

namespace {

// Query heads of one KV head that share a tile: the largest power of two
// <= 16 dividing the group size.
int32_t heads_per_tile(int32_t group) {
  int32_t g = 1;
  while (g < 16 && group % (2 * g) == 0) g *= 2;
  return g;
}

pkv_status check_heads(int32_t num_q_heads, int32_t num_kv_heads, int32_t& tile) {
  if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0)
    return fail(PKV_E_BAD_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  tile = pkv::kPrefillTileRows / heads_per_tile(num_q_heads / num_kv_heads);
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_prefill_plan_ints(const int32_t* q_lens, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t* plan_ints) {
  if (!plan_ints) return fail(PKV_E_BAD_ARG, "null plan_ints");
  if (num_seqs < 0 || (num_seqs > 0 && !q_lens)) return fail(PKV_E_BAD_ARG, "bad q_lens");
  int32_t tile = 0;
  if (pkv_status st = check_heads(num_q_heads, num_kv_heads, tile)) return st;
  int64_t work = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (q_lens[i] < 1) return fail(PKV_E_BAD_ARG, "every q_len must be >= 1");
    work += (int64_t(q_lens[i]) + tile - 1) / tile;
  }
  const int64_t total = 2 * work + num_seqs + 1;
  if (total > INT32_MAX) return fail(PKV_E_BAD_ARG, "plan too large");
  *plan_ints = int32_t(total);
  return PKV_OK;
}

pkv_status pkv_prefill_plan(const int32_t* q_lens, const int32_t* context_lens, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t* plan, int32_t cap,
                            pkv_prefill_plan_info* info) {
  if (!info) return fail(PKV_E_BAD_ARG, "null info");
  if (num_seqs < 0 || (num_seqs > 0 && (!q_lens || !context_lens)))
    return fail(PKV_E_BAD_ARG, "bad q_lens / context_lens");
  int32_t tile = 0;
  if (pkv_status st = check_heads(num_q_heads, num_kv_heads, tile)) return st;
  int64_t work = 0, total_q = 0;
  int32_t max_len = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (q_lens[i] < 1) return fail(PKV_E_BAD_ARG, "every q_len must be >= 1");
    if (context_lens[i] < q_lens[i])
      return fail(PKV_E_BAD_ARG, "a context is shorter than its chunk of queries");
    work += (int64_t(q_lens[i]) + tile - 1) / tile;
    total_q += q_lens[i];
    max_len = std::max(max_len, context_lens[i]);
  }
  const int64_t need = 2 * work + num_seqs + 1;
  if (need > INT32_MAX || total_q > INT32_MAX) return fail(PKV_E_BAD_ARG, "plan too large");
  if (cap < need || !plan) return fail(PKV_E_BAD_ARG, "plan buffer too small");

  // items with their cost (keys attended by the tile's last query)
  thread_local std::vector<int64_t> key;
  thread_local std::vector<int32_t> order, item_seq, item_tile;
  key.clear();
  item_seq.clear();
  item_tile.clear();
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t C = context_lens[i] - q_lens[i];
    for (int32_t t0 = 0, j = 0; t0 < q_lens[i]; t0 += tile, ++j) {
      key.push_back(int64_t(C) + std::min(t0 + tile, q_lens[i]));
      item_seq.push_back(i);
      item_tile.push_back(j);
    }
  }
  order.resize(key.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [](int32_t a, int32_t b) { return key[a] > key[b]; });
  for (size_t w = 0; w < order.size(); ++w) {
    plan[2 * w] = item_seq[order[w]];
    plan[2 * w + 1] = item_tile[order[w]];
  }
  int32_t* q_start = plan + 2 * work;
  q_start[0] = 0;
  for (int32_t i = 0; i < num_seqs; ++i) q_start[i + 1] = q_start[i] + q_lens[i];

  info->num_seqs = num_seqs;
  info->num_q_heads = num_q_heads;
  info->num_kv_heads = num_kv_heads;
  info->tile_tokens = tile;
  info->n_work = int32_t(work);
  info->total_q = int32_t(total_q);
  info->max_context_len = max_len;
  info->plan_ints = int32_t(need);
  return PKV_OK;
}

}  // extern "C"
