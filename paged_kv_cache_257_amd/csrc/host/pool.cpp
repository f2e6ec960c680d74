// Host block allocator of libpkv (CPU only; builds with g++ or hipcc).
//
// Follows "04 — Hacia PagedAttention (vista previa)", section "La idea de
// PagedAttention", steps 1-4 (fixed-size blocks, one block table per
// sequence, append into the last block or a newly taken one, free back to a
// free list) and "PagedAttention e continuous batching", 01 · Conceito,
// paragraph 6 (shared read-only blocks, copy-on-write for the writer of a
// diverging branch, reference counts deciding when a block returns to the
// pool) and paragraph 7 (admission decided in blocks, failing up front).
//
// Policy choices the pages leave open, fixed so that tables are
// reproducible bit for bit:
//   * the free list is a stack seeded with free_order (free_order[0] first);
//   * freeing walks a table front to back;
//   * copy-on-write happens on the first token written into a partly filled
//     last block whose refcount is above one; a full block is never copied;
//   * every call is all-or-nothing: a dry run checks ids, table capacity and
//     the number of free blocks first, then the state is changed.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>

#include "pool_internal.h"

namespace {
thread_local std::string g_last_error;
}

namespace pkv {

pkv_status fail(pkv_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

pkv_status ok() { return PKV_OK; }

}  // namespace pkv

using pkv::fail;

extern "C" const char* pkv_last_error(void) { return g_last_error.c_str(); }

namespace {

using pkv::find_seq;

int64_t blocks_for(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

int32_t pop_block(pkv_pool* p) {
  int32_t b = p->free_stack.back();
  p->free_stack.pop_back();
  p->rc[b] = 1;
  return b;
}

void release_block(pkv_pool* p, int32_t b) {
  if (--p->rc[b] == 0) p->free_stack.push_back(b);
}

// Store one token at the end of s; the dry run has made sure it succeeds.
int64_t append_token(pkv_pool* p, pkv_seq_state& s) {
  const int32_t bs = p->desc.block_size;
  const int32_t L = s.length;
  if (L % bs == 0) {
    s.table.push_back(pop_block(p));
  } else {
    int32_t last = s.table.back();
    if (p->rc[last] > 1) {
      int32_t fresh = pop_block(p);
      p->cow_pending.emplace_back(last, fresh);
      p->cow_copies++;
      p->rc[last]--;
      s.table.back() = fresh;
    }
  }
  s.length = L + 1;
  return static_cast<int64_t>(s.table[L / bs]) * bs + L % bs;
}

// Dry run of appending n tokens to a sequence of (table size, length, last
// block) as the current state would do it.  `avail` is the free-block count
// still available to this call; p->rc_taken counts references of shared last
// blocks already given up earlier in the same call (p->rc_touched lists the
// entries to clear afterwards).
pkv_status dry_append(pkv_pool* p, size_t table_size, int32_t length, int32_t last_block, int32_t n,
                      int64_t& avail) {
  const int32_t bs = p->desc.block_size;
  if (n == 0) return PKV_OK;
  if (length % bs != 0) {
    int32_t& taken = p->rc_taken[last_block];
    if (p->rc[last_block] - taken > 1) {
      if (avail == 0) return fail(PKV_E_NO_BLOCKS, "no free block for copy-on-write");
      avail--;
      if (taken++ == 0) p->rc_touched.push_back(last_block);
    }
  }
  // new blocks opened at positions that start a block; the token-by-token
  // order decides which error comes first: a boundary checks table capacity,
  // then free blocks
  const int64_t opened = blocks_for(int64_t(length) + n, bs) - blocks_for(length, bs);
  if (opened > 0) {
    const int64_t room = p->desc.max_blocks_per_seq - int64_t(table_size);
    const int64_t can = std::min<int64_t>(room, avail);
    if (can < opened) {
      if (room <= avail) return fail(PKV_E_TABLE_FULL, "block table is full");
      return fail(PKV_E_NO_BLOCKS, "no free block");
    }
    avail -= opened;
  }
  return PKV_OK;
}

void clear_dry_run(pkv_pool* p) {
  for (int32_t b : p->rc_touched) p->rc_taken[b] = 0;
  p->rc_touched.clear();
}

pkv_status check_pool(const pkv_pool* p) {
  if (!p) return fail(PKV_E_BAD_ARG, "null pool");
  return PKV_OK;
}

// A new live sequence with the next id; returns its state.
pkv_seq_state& new_seq(pkv_pool* p) {
  int32_t slot;
  if (!p->free_slots.empty()) {
    slot = p->free_slots.back();
    p->free_slots.pop_back();
  } else {
    slot = int32_t(p->slots.size());
    p->slots.emplace_back();
  }
  pkv_seq_state& s = p->slots[slot];
  s.id = p->next_id++;
  s.length = 0;
  s.table.clear();
  s.mark = 0;
  p->index.insert(s.id, slot);
  p->live++;
  return s;
}

std::string unknown(int32_t id) { return "unknown sequence " + std::to_string(id); }

}  // namespace

extern "C" {

pkv_status pkv_pool_create(const pkv_pool_desc* desc, void* k_cache, void* v_cache,
                           const int32_t* free_order, pkv_pool** out) {
  if (!desc || !out) return fail(PKV_E_BAD_ARG, "null desc or out");
  const pkv_pool_desc& d = *desc;
  if (d.num_blocks < 0 || d.block_size < 1 || d.num_kv_heads < 1 || d.head_dim < 1 ||
      d.max_blocks_per_seq < 1)
    return fail(PKV_E_BAD_ARG, "bad pool geometry");
  if (d.dtype != PKV_F32 && d.dtype != PKV_F16 && d.dtype != PKV_BF16)
    return fail(PKV_E_BAD_ARG, "bad dtype");
  if ((k_cache == nullptr) != (v_cache == nullptr))
    return fail(PKV_E_BAD_ARG, "k_cache and v_cache must both be set or both be NULL");
  if ((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) & 15)
    return fail(PKV_E_BAD_ARG, "k_cache and v_cache must be 16-byte aligned (the kernels move 16-byte chunks)");
  std::vector<int32_t> order(d.num_blocks);
  if (free_order) {
    std::vector<char> seen(d.num_blocks, 0);
    for (int32_t i = 0; i < d.num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= d.num_blocks || seen[b])
        return fail(PKV_E_BAD_ARG, "free_order is not a permutation of the block ids");
      seen[b] = 1;
      order[i] = b;
    }
  } else {
    for (int32_t i = 0; i < d.num_blocks; ++i) order[i] = i;
  }
  pkv_pool* p = new (std::nothrow) pkv_pool();
  if (!p) return fail(PKV_E_BAD_ARG, "out of host memory");
  p->desc = d;
  p->k_cache = k_cache;
  p->v_cache = v_cache;
  p->initial_order = std::move(order);
  p->rc_taken.assign(d.num_blocks, 0);
  pkv_pool_reset(p);
  *out = p;
  return PKV_OK;
}

pkv_status pkv_pool_destroy(pkv_pool* pool) {
  delete pool;
  return PKV_OK;
}

pkv_status pkv_pool_reset(pkv_pool* p) {
  if (pkv_status st = check_pool(p)) return st;
  p->free_stack.assign(p->initial_order.rbegin(), p->initial_order.rend());
  p->rc.assign(p->desc.num_blocks, 0);
  p->slots.clear();
  p->free_slots.clear();
  p->index.clear();
  p->live = 0;
  p->next_id = 0;
  p->cow_pending.clear();
  p->alloc_failures = p->cow_copies = p->forks = 0;
  return PKV_OK;
}

pkv_status pkv_pool_get_desc(const pkv_pool* p, pkv_pool_desc* out) {
  if (pkv_status st = check_pool(p)) return st;
  if (!out) return fail(PKV_E_BAD_ARG, "null out");
  *out = p->desc;
  return PKV_OK;
}

pkv_status pkv_seq_alloc(pkv_pool* p, int32_t n_tokens, int32_t* seq, int64_t* slots) {
  if (pkv_status st = check_pool(p)) return st;
  if (!seq || n_tokens < 0) return fail(PKV_E_BAD_ARG, "null seq or negative token count");
  int64_t avail = int64_t(p->free_stack.size());
  pkv_status st = dry_append(p, 0, 0, -1, n_tokens, avail);
  clear_dry_run(p);
  if (st != PKV_OK) {
    if (st == PKV_E_NO_BLOCKS) p->alloc_failures++;
    return st;
  }
  pkv_seq_state& s = new_seq(p);
  s.table.reserve(size_t(blocks_for(n_tokens, p->desc.block_size)));
  for (int32_t t = 0; t < n_tokens; ++t) {
    int64_t slot = append_token(p, s);
    if (slots) slots[t] = slot;
  }
  *seq = s.id;
  return PKV_OK;
}

pkv_status pkv_seq_append_batch(pkv_pool* p, const int32_t* seqs, int32_t n_seqs, int32_t n_tokens,
                                int64_t* slots) {
  if (pkv_status st = check_pool(p)) return st;
  if (n_seqs < 0 || n_tokens < 0 || (n_seqs > 0 && !seqs))
    return fail(PKV_E_BAD_ARG, "bad batch arguments");
  // duplicates: mark every live sequence with this call's epoch; ids that
  // are not live (the call fails anyway) are checked by sorting
  const uint64_t epoch = ++p->epoch;
  bool any_unknown = false;
  for (int32_t i = 0; i < n_seqs; ++i) {
    pkv_seq_state* s = find_seq(p, seqs[i]);
    if (!s) {
      any_unknown = true;
    } else {
      if (s->mark == epoch) return fail(PKV_E_BAD_ARG, "duplicate sequence in batch");
      s->mark = epoch;
    }
  }
  if (any_unknown) {
    std::vector<int32_t> sorted(seqs, seqs + n_seqs);
    std::sort(sorted.begin(), sorted.end());
    if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
      return fail(PKV_E_BAD_ARG, "duplicate sequence in batch");
  }
  int64_t avail = int64_t(p->free_stack.size());
  for (int32_t i = 0; i < n_seqs; ++i) {
    const pkv_seq_state* s = find_seq(p, seqs[i]);
    pkv_status st = s ? PKV_OK : fail(PKV_E_BAD_SEQ, unknown(seqs[i]));
    if (st == PKV_OK) {
      const int32_t last = s->table.empty() ? -1 : s->table.back();
      st = dry_append(p, s->table.size(), s->length, last, n_tokens, avail);
    }
    if (st != PKV_OK) {
      clear_dry_run(p);
      if (st == PKV_E_NO_BLOCKS) p->alloc_failures++;
      return st;
    }
  }
  clear_dry_run(p);
  for (int32_t i = 0; i < n_seqs; ++i) {
    pkv_seq_state& s = *find_seq(p, seqs[i]);
    for (int32_t t = 0; t < n_tokens; ++t) {
      int64_t slot = append_token(p, s);
      if (slots) slots[int64_t(i) * n_tokens + t] = slot;
    }
  }
  return PKV_OK;
}

pkv_status pkv_seq_append(pkv_pool* p, int32_t seq, int32_t n_tokens, int64_t* slots) {
  return pkv_seq_append_batch(p, &seq, 1, n_tokens, slots);
}

pkv_status pkv_seq_fork(pkv_pool* p, int32_t parent, int32_t* child) {
  if (pkv_status st = check_pool(p)) return st;
  if (!child) return fail(PKV_E_BAD_ARG, "null child");
  if (!find_seq(p, parent)) return fail(PKV_E_BAD_SEQ, unknown(parent));
  pkv_seq_state& c = new_seq(p);  // may move `slots`: look the parent up again
  const pkv_seq_state& par = *find_seq(p, parent);
  c.table = par.table;
  c.length = par.length;
  for (int32_t b : c.table) p->rc[b]++;
  p->forks++;
  *child = c.id;
  return PKV_OK;
}

pkv_status pkv_seq_fork_prefix(pkv_pool* p, int32_t parent, int32_t n_tokens, int32_t* child) {
  if (pkv_status st = check_pool(p)) return st;
  if (!child) return fail(PKV_E_BAD_ARG, "null child");
  const pkv_seq_state* par0 = find_seq(p, parent);
  if (!par0) return fail(PKV_E_BAD_SEQ, unknown(parent));
  if (n_tokens < 0 || n_tokens > par0->length)
    return fail(PKV_E_BAD_ARG, "prefix longer than the parent");
  pkv_seq_state& c = new_seq(p);  // may move `slots`: look the parent up again
  const pkv_seq_state& par = *find_seq(p, parent);
  const int32_t nb = int32_t(blocks_for(n_tokens, p->desc.block_size));
  c.table.assign(par.table.begin(), par.table.begin() + nb);
  c.length = n_tokens;
  for (int32_t b : c.table) p->rc[b]++;
  p->forks++;
  *child = c.id;
  return PKV_OK;
}

pkv_status pkv_seq_free(pkv_pool* p, int32_t seq) {
  if (pkv_status st = check_pool(p)) return st;
  const int32_t slot = p->index.find(seq);
  if (slot < 0) return fail(PKV_E_BAD_SEQ, unknown(seq));
  pkv_seq_state& s = p->slots[slot];
  for (int32_t b : s.table) release_block(p, b);
  s.table.clear();
  s.id = -1;
  p->index.erase(seq);
  p->free_slots.push_back(slot);
  p->live--;
  return PKV_OK;
}

pkv_status pkv_seq_free_batch(pkv_pool* p, const int32_t* seqs, int32_t n_seqs) {
  if (pkv_status st = check_pool(p)) return st;
  if (n_seqs < 0 || (n_seqs > 0 && !seqs)) return fail(PKV_E_BAD_ARG, "bad batch arguments");
  // all or nothing: every id live and none twice, checked before any is freed
  const uint64_t epoch = ++p->epoch;
  for (int32_t i = 0; i < n_seqs; ++i) {
    pkv_seq_state* s = find_seq(p, seqs[i]);
    if (!s) return fail(PKV_E_BAD_SEQ, unknown(seqs[i]));
    if (s->mark == epoch) return fail(PKV_E_BAD_ARG, "duplicate sequence in batch");
    s->mark = epoch;
  }
  for (int32_t i = 0; i < n_seqs; ++i)
    if (pkv_status st = pkv_seq_free(p, seqs[i])) return st;
  return PKV_OK;
}

pkv_status pkv_seq_fork_batch(pkv_pool* p, const int32_t* parents, int32_t n, int32_t* children) {
  if (pkv_status st = check_pool(p)) return st;
  if (n < 0 || (n > 0 && (!parents || !children))) return fail(PKV_E_BAD_ARG, "bad batch arguments");
  // all or nothing: every parent live before any child is made
  for (int32_t i = 0; i < n; ++i)
    if (!find_seq(p, parents[i])) return fail(PKV_E_BAD_SEQ, unknown(parents[i]));
  for (int32_t i = 0; i < n; ++i)
    if (pkv_status st = pkv_seq_fork(p, parents[i], children + i)) return st;
  return PKV_OK;
}

pkv_status pkv_seq_length(const pkv_pool* p, int32_t seq, int32_t* length) {
  if (pkv_status st = check_pool(p)) return st;
  if (!length) return fail(PKV_E_BAD_ARG, "null length");
  const pkv_seq_state* s = find_seq(p, seq);
  if (!s) return fail(PKV_E_BAD_SEQ, unknown(seq));
  *length = s->length;
  return PKV_OK;
}

pkv_status pkv_seq_table(const pkv_pool* p, int32_t seq, int32_t* table, int32_t cap, int32_t* n) {
  if (pkv_status st = check_pool(p)) return st;
  if (!n || cap < 0 || (cap > 0 && !table)) return fail(PKV_E_BAD_ARG, "bad table buffer");
  const pkv_seq_state* s = find_seq(p, seq);
  if (!s) return fail(PKV_E_BAD_SEQ, unknown(seq));
  const auto& t = s->table;
  *n = int32_t(t.size());
  if (int64_t(t.size()) > cap) return fail(PKV_E_BAD_ARG, "table buffer too small");
  std::copy(t.begin(), t.end(), table);
  return PKV_OK;
}

pkv_status pkv_seq_slots(const pkv_pool* p, int32_t seq, int32_t first, int32_t n, int64_t* slots) {
  if (pkv_status st = check_pool(p)) return st;
  const pkv_seq_state* s = find_seq(p, seq);
  if (!s) return fail(PKV_E_BAD_SEQ, unknown(seq));
  if (first < 0 || n < 0 || int64_t(first) + n > s->length)
    return fail(PKV_E_BAD_ARG, "positions outside the sequence");
  if (n > 0 && !slots) return fail(PKV_E_BAD_ARG, "null slots");
  const int32_t bs = p->desc.block_size;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t pos = first + i;
    slots[i] = int64_t(s->table[size_t(pos / bs)]) * bs + pos % bs;
  }
  return PKV_OK;
}

pkv_status pkv_live_seqs(const pkv_pool* p, int32_t* ids, int32_t cap, int32_t* n) {
  if (pkv_status st = check_pool(p)) return st;
  if (!n || cap < 0 || (cap > 0 && !ids)) return fail(PKV_E_BAD_ARG, "bad id buffer");
  *n = p->live;
  if (p->live > cap) return fail(PKV_E_BAD_ARG, "id buffer too small");
  int32_t i = 0;
  for (const pkv_seq_state& s : p->slots)
    if (s.id >= 0) ids[i++] = s.id;
  std::sort(ids, ids + i);
  return PKV_OK;
}

pkv_status pkv_free_list(const pkv_pool* p, int32_t* blocks, int32_t cap, int32_t* n) {
  if (pkv_status st = check_pool(p)) return st;
  if (!n || cap < 0 || (cap > 0 && !blocks)) return fail(PKV_E_BAD_ARG, "bad block buffer");
  *n = int32_t(p->free_stack.size());
  if (int64_t(p->free_stack.size()) > cap) return fail(PKV_E_BAD_ARG, "block buffer too small");
  std::copy(p->free_stack.rbegin(), p->free_stack.rend(), blocks);
  return PKV_OK;
}

pkv_status pkv_refcounts(const pkv_pool* p, int32_t* refcounts) {
  if (pkv_status st = check_pool(p)) return st;
  if (!refcounts) return fail(PKV_E_BAD_ARG, "null refcounts");
  std::copy(p->rc.begin(), p->rc.end(), refcounts);
  return PKV_OK;
}

pkv_status pkv_stats(const pkv_pool* p, pkv_stats_t* out) {
  if (pkv_status st = check_pool(p)) return st;
  if (!out) return fail(PKV_E_BAD_ARG, "null out");
  pkv_stats_t s{};
  s.free_blocks = int64_t(p->free_stack.size());
  s.used_blocks = p->desc.num_blocks - s.free_blocks;
  s.alloc_failures = p->alloc_failures;
  const int32_t bs = p->desc.block_size;
  for (const pkv_seq_state& q : p->slots)
    if (q.id >= 0) s.tail_waste_slots += int64_t(bs) * int64_t(q.table.size()) - q.length;
  for (int32_t r : p->rc) s.shared_blocks += (r > 1);
  s.cow_copies = p->cow_copies;
  s.forks = p->forks;
  s.live_seqs = p->live;
  *out = s;
  return PKV_OK;
}

pkv_status pkv_take_cow(pkv_pool* p, int32_t* pairs, int32_t cap, int32_t* n) {
  if (pkv_status st = check_pool(p)) return st;
  if (!n || cap < 0 || (cap > 0 && !pairs)) return fail(PKV_E_BAD_ARG, "bad pair buffer");
  *n = int32_t(p->cow_pending.size());
  if (int64_t(p->cow_pending.size()) > cap) return fail(PKV_E_BAD_ARG, "pair buffer too small");
  for (size_t i = 0; i < p->cow_pending.size(); ++i) {
    pairs[2 * i] = p->cow_pending[i].first;
    pairs[2 * i + 1] = p->cow_pending[i].second;
  }
  p->cow_pending.clear();
  return PKV_OK;
}

pkv_status pkv_build_batch(const pkv_pool* p, const int32_t* seqs, int32_t n_seqs,
                           int32_t* block_tables, int32_t table_stride, int32_t* context_lens) {
  if (pkv_status st = check_pool(p)) return st;
  if (n_seqs < 0 || table_stride < 1 || (n_seqs > 0 && (!seqs || !block_tables || !context_lens)))
    return fail(PKV_E_BAD_ARG, "bad batch arguments");
  for (int32_t i = 0; i < n_seqs; ++i) {
    const pkv_seq_state* s = find_seq(p, seqs[i]);
    if (!s) return fail(PKV_E_BAD_SEQ, unknown(seqs[i]));
    if (int64_t(s->table.size()) > table_stride)
      return fail(PKV_E_BAD_ARG, "a table is wider than table_stride");
  }
  for (int32_t i = 0; i < n_seqs; ++i) {
    const pkv_seq_state& s = *find_seq(p, seqs[i]);
    int32_t* row = block_tables + int64_t(i) * table_stride;
    std::copy(s.table.begin(), s.table.end(), row);
    std::fill(row + s.table.size(), row + table_stride, -1);
    context_lens[i] = s.length;
  }
  return PKV_OK;
}

}  // extern "C"
