// pkv_utilisation: naive contiguous reservation vs this library's paged
// allocator for one set of concurrent requests (the tutorial's comparison,
// "Paged Attention em Large Language Models LLMs", opening paragraph).
#include <cstdint>

#include "pool_internal.h"

using pkv::fail;

extern "C" pkv_status pkv_utilisation(const int32_t* lengths, int32_t n, int32_t max_len,
                                      int32_t block_size, pkv_utilisation_t* out) {
  if (!out || n < 0 || (n > 0 && !lengths)) return fail(PKV_E_BAD_ARG, "bad arguments");
  if (max_len < 1 || block_size < 1) return fail(PKV_E_BAD_ARG, "bad max_len / block_size");
  int64_t blocks = 0, used = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (lengths[i] < 1 || lengths[i] > max_len)
      return fail(PKV_E_BAD_ARG, "every length must lie in [1, max_len]");
    blocks += (int64_t(lengths[i]) + block_size - 1) / block_size;
    used += lengths[i];
  }
  if (blocks > INT32_MAX) return fail(PKV_E_BAD_ARG, "too many blocks");
  pkv_pool_desc d{};
  d.num_blocks = int32_t(blocks);
  d.block_size = block_size;
  d.num_kv_heads = 1;
  d.head_dim = 1;
  d.max_blocks_per_seq = (max_len + block_size - 1) / block_size;
  d.dtype = PKV_F16;
  pkv_pool* pool = nullptr;
  if (pkv_status st = pkv_pool_create(&d, nullptr, nullptr, nullptr, &pool)) return st;
  pkv_status st = PKV_OK;
  for (int32_t i = 0; i < n && st == PKV_OK; ++i) {
    int32_t seq = -1;
    st = pkv_seq_alloc(pool, lengths[i], &seq, nullptr);
  }
  pkv_stats_t stats{};
  if (st == PKV_OK) st = pkv_stats(pool, &stats);
  pkv_pool_destroy(pool);
  if (st != PKV_OK) return st;
  out->requests = n;
  out->tokens_used = used;
  out->naive_reserved_tokens = int64_t(n) * max_len;
  out->paged_blocks = stats.used_blocks;
  out->paged_reserved_tokens = stats.used_blocks * block_size;
  out->naive_waste_tokens = out->naive_reserved_tokens - used;
  out->paged_waste_tokens = stats.tail_waste_slots;
  return PKV_OK;
}
