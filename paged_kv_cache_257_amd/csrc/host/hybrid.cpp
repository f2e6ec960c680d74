// Hybrid two-pool manager: paged K/V blocks plus fixed-size per-sequence
// state slots ("PagedAttention e continuous batching", 01 · Conceito,
// paragraph 5).  Host side; the state copy kernel lives with the device code.
#include <algorithm>
#include <string>

#include "hybrid_internal.h"

using pkv::fail;

extern "C" {

pkv_status pkv_hybrid_create(pkv_pool* kv, int32_t num_slots, int64_t slot_bytes, void* state_base,
                             const int32_t* slot_order, pkv_hybrid** out) {
  if (!kv || !out) return fail(PKV_E_BAD_ARG, "null pool or out");
  if (num_slots < 0 || slot_bytes < 16 || slot_bytes % 16 != 0)
    return fail(PKV_E_BAD_ARG, "num_slots >= 0 and slot_bytes a positive multiple of 16");
  std::vector<int32_t> order(num_slots);
  if (slot_order) {
    std::vector<char> seen(num_slots, 0);
    for (int32_t i = 0; i < num_slots; ++i) {
      const int32_t s = slot_order[i];
      if (s < 0 || s >= num_slots || seen[s])
        return fail(PKV_E_BAD_ARG, "slot_order is not a permutation of the slot ids");
      seen[s] = 1;
      order[i] = s;
    }
  } else {
    for (int32_t i = 0; i < num_slots; ++i) order[i] = i;
  }
  pkv_hybrid* h = new (std::nothrow) pkv_hybrid();
  if (!h) return fail(PKV_E_BAD_ARG, "out of host memory");
  h->kv = kv;
  h->num_slots = num_slots;
  h->slot_bytes = slot_bytes;
  h->state_base = state_base;
  h->free_slots.assign(order.rbegin(), order.rend());  // order[0] on top
  *out = h;
  return pkv::ok();
}

pkv_status pkv_hybrid_destroy(pkv_hybrid* h) {
  delete h;
  return pkv::ok();
}

pkv_status pkv_hybrid_admit(pkv_hybrid* h, int32_t n_tokens, int32_t* seq, int32_t* slot,
                            int64_t* slots) {
  if (!h || !seq || !slot) return fail(PKV_E_BAD_ARG, "null argument");
  if (h->free_slots.empty()) {
    h->refusals++;
    return fail(PKV_E_NO_SLOTS, "no free state slot");
  }
  if (pkv_status st = pkv_seq_alloc(h->kv, n_tokens, seq, slots)) {
    if (st == PKV_E_NO_BLOCKS || st == PKV_E_TABLE_FULL) h->refusals++;
    return st;
  }
  *slot = h->free_slots.back();
  h->free_slots.pop_back();
  h->slot_of[*seq] = *slot;
  return pkv::ok();
}

pkv_status pkv_hybrid_fork(pkv_hybrid* h, int32_t parent, int32_t* child, int32_t* child_slot) {
  if (!h || !child || !child_slot) return fail(PKV_E_BAD_ARG, "null argument");
  auto it = h->slot_of.find(parent);
  if (it == h->slot_of.end())
    return fail(PKV_E_BAD_SEQ, "sequence " + std::to_string(parent) + " is not held by this manager");
  if (h->free_slots.empty()) {
    h->refusals++;
    return fail(PKV_E_NO_SLOTS, "no free state slot");
  }
  const int32_t pslot = it->second;
  if (pkv_status st = pkv_seq_fork(h->kv, parent, child)) return st;
  *child_slot = h->free_slots.back();
  h->free_slots.pop_back();
  h->slot_of[*child] = *child_slot;
  h->copies.emplace_back(pslot, *child_slot);
  h->state_copies++;
  return pkv::ok();
}

pkv_status pkv_hybrid_free(pkv_hybrid* h, int32_t seq) {
  if (!h) return fail(PKV_E_BAD_ARG, "null manager");
  auto it = h->slot_of.find(seq);
  if (it == h->slot_of.end())
    return fail(PKV_E_BAD_SEQ, "sequence " + std::to_string(seq) + " is not held by this manager");
  if (pkv_status st = pkv_seq_free(h->kv, seq)) return st;
  h->free_slots.push_back(it->second);
  h->slot_of.erase(it);
  return pkv::ok();
}

pkv_status pkv_hybrid_slot(const pkv_hybrid* h, int32_t seq, int32_t* slot) {
  if (!h || !slot) return fail(PKV_E_BAD_ARG, "null argument");
  auto it = h->slot_of.find(seq);
  if (it == h->slot_of.end()) return fail(PKV_E_BAD_SEQ, "sequence not held by this manager");
  *slot = it->second;
  return pkv::ok();
}

pkv_status pkv_hybrid_take_copies(pkv_hybrid* h, int32_t* pairs, int32_t cap, int32_t* n) {
  if (!h || !n) return fail(PKV_E_BAD_ARG, "null argument");
  const int32_t k = int32_t(h->copies.size());
  *n = k;
  if (!pairs || cap < k) return pkv::ok();
  for (int32_t i = 0; i < k; ++i) {
    pairs[2 * i] = h->copies[i].first;
    pairs[2 * i + 1] = h->copies[i].second;
  }
  h->copies.clear();
  return pkv::ok();
}

pkv_status pkv_hybrid_stats(const pkv_hybrid* h, pkv_hybrid_stats_t* out) {
  if (!h || !out) return fail(PKV_E_BAD_ARG, "null argument");
  out->free_slots = int64_t(h->free_slots.size());
  out->used_slots = int64_t(h->slot_of.size());
  out->refusals = h->refusals;
  out->state_copies = h->state_copies;
  return pkv::ok();
}

pkv_status pkv_hybrid_plan(int64_t budget_bytes, int64_t block_bytes, int32_t block_size,
                           int64_t slot_bytes, int64_t session_tokens, int32_t* sessions,
                           int32_t* num_blocks, int32_t* num_slots) {
  if (!sessions || !num_blocks || !num_slots) return fail(PKV_E_BAD_ARG, "null argument");
  if (budget_bytes < 0 || block_bytes < 1 || block_size < 1 || slot_bytes < 0 || session_tokens < 0)
    return fail(PKV_E_BAD_ARG, "bad budget arguments");
  const int64_t per = (session_tokens + block_size - 1) / block_size * block_bytes + slot_bytes;
  if (per < 1) return fail(PKV_E_BAD_ARG, "a session costs nothing");
  const int64_t n = budget_bytes / per;
  const int64_t blocks = (budget_bytes - n * slot_bytes) / block_bytes;
  if (n > INT32_MAX || blocks > INT32_MAX) return fail(PKV_E_BAD_ARG, "pools too large");
  *sessions = int32_t(n);
  *num_slots = int32_t(n);
  *num_blocks = int32_t(blocks);
  return pkv::ok();
}

}  // extern "C"
