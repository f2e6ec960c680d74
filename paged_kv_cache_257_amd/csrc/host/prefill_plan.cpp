// Host work list of a chunked-prefill launch (pkv_prefill_plan).
//
// The lesson's scheduler slices long prefills into chunks ("PagedAttention
// e continuous batching", 01 · Conceito, the scheduler paragraph); a launch
// takes one chunk of each of several sequences.  Work items are tiles of
// consecutive query tokens; a tile's cost is the number of keys its last
// token attends, so items are sorted by that, largest first, and the
// in-order workgroup dispatcher fills the tail of the launch with the
// cheap ones (a launch that runs in one round instead pairs long and short
// items on each CU).
#include <algorithm>
#include <cstdlib>
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

namespace {

constexpr int32_t kStageTokens = 32;  // keys per kernel stage
// max_keys < 0: split only launches that would leave the GPU under-filled
// (fewer than this many workgroups), into about this many.
// PKV_PREFILL_SPLIT_WGS overrides it for tuning sweeps (read per plan).
constexpr int64_t kAutoSplitWorkgroups = 512;
// Two workgroups on each of MI355X's 256 CUs: a launch of at most this many
// runs in one round.
constexpr int64_t kOneRoundWorkgroups = 512;
int64_t auto_split_workgroups() {
  const char* s = std::getenv("PKV_PREFILL_SPLIT_WGS");
  const long v = s ? std::atol(s) : 0;
  return v >= 64 && v <= 65536 ? v : kAutoSplitWorkgroups;
}
constexpr int32_t kAutoSplitMinKeys = 1024;

// Query-head groups per KV head times KV heads: workgroups per tile.
int64_t workgroups_per_tile(int32_t num_q_heads, int32_t num_kv_heads, int32_t tile) {
  const int32_t gw = pkv::kPrefillTileRows / tile;
  return int64_t(num_kv_heads) * (num_q_heads / num_kv_heads / gw);
}

// The key limit for max_keys < 0 (0: no split).
int32_t auto_max_keys(const int32_t* q_lens, const int32_t* context_lens, int32_t n, int32_t tile,
                      int64_t per_tile) {
  int64_t tiles = 0, keys = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t C = context_lens[i] - q_lens[i];
    for (int32_t t0 = 0; t0 < q_lens[i]; t0 += tile) {
      tiles++;
      keys += int64_t(C) + std::min(t0 + tile, q_lens[i]);
    }
  }
  const int64_t target = auto_split_workgroups();
  if (tiles * per_tile >= target || tiles == 0) return 0;
  const int64_t items = (target + per_tile - 1) / per_tile;
  const int64_t per_item = (keys + items - 1) / items;
  return int32_t(std::max<int64_t>(kAutoSplitMinKeys, (per_item + kStageTokens - 1) / kStageTokens * kStageTokens));
}

struct Counts {
  int64_t work = 0, split = 0, partials = 0, total_q = 0;
  int32_t max_len = 0;
};

// Parts of a tile whose last query attends `keys` keys.
int32_t parts_for(int64_t keys, int32_t max_keys) {
  if (max_keys <= 0 || keys <= max_keys) return 1;
  const int64_t stages = (keys + kStageTokens - 1) / kStageTokens;
  const int64_t per = std::max<int64_t>(1, max_keys / kStageTokens);
  return int32_t((stages + per - 1) / per);
}

pkv_status count(const int32_t* q_lens, const int32_t* context_lens, int32_t n, int32_t tile,
                 int32_t max_keys, Counts& c) {
  for (int32_t i = 0; i < n; ++i) {
    if (q_lens[i] < 1) return fail(PKV_E_BAD_ARG, "every q_len must be >= 1");
    if (context_lens && context_lens[i] < q_lens[i])
      return fail(PKV_E_BAD_ARG, "a context is shorter than its chunk of queries");
    const int32_t C = context_lens ? context_lens[i] - q_lens[i] : 0;
    for (int32_t t0 = 0; t0 < q_lens[i]; t0 += tile) {
      const int32_t parts = context_lens ? parts_for(int64_t(C) + std::min(t0 + tile, q_lens[i]), max_keys) : 1;
      c.work += parts;
      if (parts > 1) {
        c.split++;
        c.partials += parts;
      }
    }
    c.total_q += q_lens[i];
    if (context_lens) c.max_len = std::max(c.max_len, context_lens[i]);
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_prefill_plan_ints(const int32_t* q_lens, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t max_keys, int32_t* plan_ints) {
  if (!plan_ints) return fail(PKV_E_BAD_ARG, "null plan_ints");
  if (num_seqs < 0 || (num_seqs > 0 && (!q_lens || !context_lens)))
    return fail(PKV_E_BAD_ARG, "bad q_lens / context_lens");
  int32_t tile = 0;
  if (pkv_status st = check_heads(num_q_heads, num_kv_heads, tile)) return st;
  Counts c;
  if (pkv_status st = count(q_lens, context_lens, num_seqs, tile, 0, c)) return st;  // validates
  if (max_keys < 0)
    max_keys = auto_max_keys(q_lens, context_lens, num_seqs, tile,
                             workgroups_per_tile(num_q_heads, num_kv_heads, tile));
  c = Counts();
  if (pkv_status st = count(q_lens, context_lens, num_seqs, tile, max_keys, c)) return st;
  const int64_t total = 6 * c.work + num_seqs + 1 + 2 * c.split;
  if (total > INT32_MAX) return fail(PKV_E_BAD_ARG, "plan too large");
  *plan_ints = int32_t(total);
  return PKV_OK;
}

pkv_status pkv_prefill_plan(const int32_t* q_lens, const int32_t* context_lens, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t max_keys,
                            int32_t* plan, int32_t cap, pkv_prefill_plan_info* info) {
  if (!info) return fail(PKV_E_BAD_ARG, "null info");
  if (num_seqs < 0 || (num_seqs > 0 && (!q_lens || !context_lens)))
    return fail(PKV_E_BAD_ARG, "bad q_lens / context_lens");
  int32_t tile = 0;
  if (pkv_status st = check_heads(num_q_heads, num_kv_heads, tile)) return st;
  Counts c;
  if (pkv_status st = count(q_lens, context_lens, num_seqs, tile, 0, c)) return st;  // validates
  if (max_keys < 0)
    max_keys = auto_max_keys(q_lens, context_lens, num_seqs, tile,
                             workgroups_per_tile(num_q_heads, num_kv_heads, tile));
  c = Counts();
  if (pkv_status st = count(q_lens, context_lens, num_seqs, tile, max_keys, c)) return st;
  const int64_t need = 6 * c.work + num_seqs + 1 + 2 * c.split;
  if (need > INT32_MAX || c.total_q > INT32_MAX || c.partials > INT32_MAX)
    return fail(PKV_E_BAD_ARG, "plan too large");
  if (cap < need || !plan) return fail(PKV_E_BAD_ARG, "plan buffer too small");

  // items with their cost (keys they attend), then sorted largest first
  struct Item {
    int32_t seq, tile, s0, s1, split, part;
    int64_t keys;
  };
  thread_local std::vector<Item> items;
  thread_local std::vector<int32_t> order;
  items.clear();
  int32_t* split_tab = plan + 6 * c.work + num_seqs + 1;
  int32_t n_split = 0, n_partials = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t C = context_lens[i] - q_lens[i];
    for (int32_t t0 = 0, j = 0; t0 < q_lens[i]; t0 += tile, ++j) {
      const int64_t keys = int64_t(C) + std::min(t0 + tile, q_lens[i]);
      const int32_t stages = int32_t((keys + kStageTokens - 1) / kStageTokens);
      const int32_t parts = parts_for(keys, max_keys);
      if (parts == 1) {
        items.push_back({i, j, 0, stages, -1, 0, keys});
        continue;
      }
      // even split: part q covers stages [q S / P, (q + 1) S / P), sizes
      // differ by at most one and none exceeds max_keys
      split_tab[2 * n_split] = n_partials;
      split_tab[2 * n_split + 1] = parts;
      for (int32_t q = 0; q < parts; ++q) {
        const int32_t s0 = int32_t(int64_t(q) * stages / parts);
        const int32_t s1 = int32_t(int64_t(q + 1) * stages / parts);
        items.push_back({i, j, s0, s1, n_split, q, int64_t(s1 - s0) * kStageTokens});
      }
      n_partials += parts;
      n_split++;
    }
  }
  order.resize(items.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [](int32_t a, int32_t b) { return items[a].keys > items[b].keys; });
  // A launch of at most two workgroups per CU runs in one round: the
  // dispatcher gives each CU workgroup j and j + 256 (the XCDs take
  // workgroups in turn and fill their CUs breadth first), so the second
  // half of the items goes in ascending order and every CU holds a long and
  // a short tile of about the same total (the causal tiles of one chunk
  // differ in length by the chunk).
  if (int64_t(order.size()) * workgroups_per_tile(num_q_heads, num_kv_heads, tile) <= kOneRoundWorkgroups)
    std::reverse(order.begin() + order.size() / 2, order.end());
  for (size_t w = 0; w < order.size(); ++w) {
    const Item& it = items[order[w]];
    int32_t* e = plan + 6 * w;
    e[0] = it.seq;
    e[1] = it.tile;
    e[2] = it.s0;
    e[3] = it.s1;
    e[4] = it.split;
    e[5] = it.part;
  }
  int32_t* q_start = plan + 6 * c.work;
  q_start[0] = 0;
  for (int32_t i = 0; i < num_seqs; ++i) q_start[i + 1] = q_start[i] + q_lens[i];

  info->num_seqs = num_seqs;
  info->num_q_heads = num_q_heads;
  info->num_kv_heads = num_kv_heads;
  info->tile_tokens = tile;
  info->n_work = int32_t(c.work);
  info->total_q = int32_t(c.total_q);
  info->max_context_len = c.max_len;
  info->plan_ints = int32_t(need);
  info->n_split = n_split;
  info->n_partials = n_partials;
  return PKV_OK;
}

size_t pkv_prefill_workspace_bytes(const pkv_prefill_plan_info* info, int32_t head_dim) {
  if (!info || head_dim < 1 || info->num_kv_heads < 1 || info->n_split <= 0) return 0;
  const int32_t hgroups = info->num_q_heads / info->num_kv_heads /
                          (pkv::kPrefillTileRows / info->tile_tokens) * info->num_kv_heads;
  const size_t tickets = (size_t(info->n_split) * hgroups * 4 + 255) / 256 * 256;
  const size_t record = ((size_t(head_dim) + 2) * sizeof(float) + 127) / 128 * 128;
  return tickets + size_t(info->n_partials) * hgroups * pkv::kPrefillTileRows * record;
}

}  // extern "C"
