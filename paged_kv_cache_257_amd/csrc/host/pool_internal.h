// Internal state of a pkv_pool, shared by the host allocator and the device
// entry points.  Plain C++17: no HIP types, builds with g++ alone.
#pragma once

#include <cstdint>
#include <string>
#include <utility>
#include <vector>

#include "pkv.h"

struct pkv_seq_state {
  std::vector<int32_t> table;  // physical block of each logical block
  int32_t length = 0;          // tokens stored
  int32_t id = -1;             // -1: the slot is free
  uint64_t mark = 0;           // batch epoch that last touched the sequence
};

namespace pkv {

// Open-addressing map from sequence id to slot index (linear probing,
// power-of-two capacity, tombstones on erase).  Lookups touch one or two
// cache lines; no allocation except when the table grows.
class SeqIndex {
 public:
  int32_t find(int32_t id) const {
    if (cap_ == 0) return -1;
    for (uint32_t i = hash(id);; i = (i + 1) & (cap_ - 1)) {
      const Entry& e = e_[i];
      if (e.key == id) return e.val;
      if (e.key == kEmpty) return -1;
    }
  }
  void insert(int32_t id, int32_t slot) {
    if ((size_ + tombs_ + 1) * 2 > cap_) rehash(cap_ == 0 ? 64 : (size_ + 1) * 4 > cap_ ? cap_ * 2 : cap_);
    uint32_t i = hash(id);
    while (e_[i].key != kEmpty && e_[i].key != kTomb) i = (i + 1) & (cap_ - 1);
    if (e_[i].key == kTomb) tombs_--;
    e_[i] = {id, slot};
    size_++;
  }
  void erase(int32_t id) {
    for (uint32_t i = hash(id);; i = (i + 1) & (cap_ - 1)) {
      if (e_[i].key == id) {
        e_[i].key = kTomb;
        size_--;
        tombs_++;
        return;
      }
      if (e_[i].key == kEmpty) return;
    }
  }
  void clear() {
    e_.assign(e_.size(), Entry{kEmpty, 0});
    size_ = tombs_ = 0;
  }

 private:
  static constexpr int32_t kEmpty = -1, kTomb = -2;
  struct Entry {
    int32_t key, val;
  };
  uint32_t hash(int32_t id) const { return (uint32_t(id) * 2654435761u) & (cap_ - 1); }
  void rehash(uint32_t cap) {
    std::vector<Entry> old(std::move(e_));
    e_.assign(cap, Entry{kEmpty, 0});
    cap_ = cap;
    size_ = tombs_ = 0;
    for (const Entry& e : old)
      if (e.key >= 0) insert(e.key, e.val);
  }
  std::vector<Entry> e_;
  uint32_t cap_ = 0, size_ = 0, tombs_ = 0;
};

}  // namespace pkv

struct pkv_pool {
  pkv_pool_desc desc{};
  void* k_cache = nullptr;  // device, [num_blocks][H_kv][block_size][head_dim]
  void* v_cache = nullptr;
  std::vector<int32_t> initial_order;        // free_order as given
  std::vector<int32_t> free_stack;           // back() is handed out next
  std::vector<int32_t> rc;                   // reference count per block
  std::vector<pkv_seq_state> slots;          // sequence states, recycled
  std::vector<int32_t> free_slots;           // unused entries of `slots`
  pkv::SeqIndex index;                       // live sequence id -> slot
  int32_t live = 0;                          // live sequences
  int32_t next_id = 0;
  uint64_t epoch = 0;                        // batch calls, for duplicate marks
  std::vector<std::pair<int32_t, int32_t>> cow_pending;  // (src, dst)
  std::vector<int32_t> rc_taken;             // dry-run scratch, all zero between calls
  std::vector<int32_t> rc_touched;
  int64_t alloc_failures = 0;
  int64_t cow_copies = 0;
  int64_t forks = 0;
};

namespace pkv {

// Record a message for pkv_last_error() and return the status.
pkv_status fail(pkv_status st, const std::string& msg);
pkv_status ok();

inline int dtype_bytes(int32_t dt) { return dt == PKV_F32 ? 4 : 2; }

// Split-K partition length used when a caller passes partition_tokens = 0.
// 2048 tokens (128 blocks of 16): measured best or within 1% of best for
// 2k-4k-token batches of 32 KV heads in 16-bit types on MI355X; shorter
// partitions add combine work and more workgroups than the chip needs.
constexpr int32_t kDefaultPartitionTokens = 2048;

// A partition_tokens argument as the size buffers are dimensioned for: 0 is
// the default, PKV_PARTITION_FILL the smallest size fill mode picks.
inline int32_t sizing_partition(int32_t P) {
  return P == 0 ? kDefaultPartitionTokens : P == PKV_PARTITION_FILL ? PKV_FILL_MIN_TOKENS : P;
}

// Query rows (token, head pairs) of one chunked-prefill workgroup: four
// waves of two 16-row groups each.
constexpr int32_t kPrefillTileRows = 128;

// Split-K plan over each sequence's private blocks (plan.cpp).
pkv_status fill_private_plan(const int32_t* lens, int32_t n, int32_t bs, int32_t P,
                             const int32_t* first_block, const int32_t* n_shared, int32_t* plan,
                             int64_t cap, pkv_decode_plan_info* info);

// Shared-block plan of a batch of live sequences (plan_shared.cpp): lens and
// shared_kv out; see pkv_decode_plan_shared.
pkv_status build_shared_plan(const pkv_pool* p, const int32_t* seqs, int32_t n, int32_t P,
                             int32_t num_q_heads, int32_t chunk_tokens, int32_t* plan, int64_t cap,
                             pkv_decode_plan_info* info);

// Upper bound of the ints build_shared_plan writes for n sequences whose
// tables hold at most the given total of blocks.
int64_t shared_plan_bound(int64_t n, int64_t total_blocks, int32_t pblocks);

// Live sequence with this id, or null.
inline pkv_seq_state* find_seq(pkv_pool* p, int32_t id) {
  const int32_t s = p->index.find(id);
  return s < 0 ? nullptr : &p->slots[s];
}
inline const pkv_seq_state* find_seq(const pkv_pool* p, int32_t id) {
  const int32_t s = p->index.find(id);
  return s < 0 ? nullptr : &p->slots[s];
}

}  // namespace pkv
