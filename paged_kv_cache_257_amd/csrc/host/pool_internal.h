// Internal state of a pkv_pool, shared by the host allocator and the device
// entry points.  Plain C++17: no HIP types, builds with g++ alone.
#pragma once

#include <cstdint>
#include <map>
#include <string>
#include <utility>
#include <vector>

#include "pkv.h"

struct pkv_seq_state {
  std::vector<int32_t> table;  // physical block of each logical block
  int32_t length = 0;          // tokens stored
};

struct pkv_pool {
  pkv_pool_desc desc{};
  void* k_cache = nullptr;  // device, [num_blocks][H_kv][block_size][head_dim]
  void* v_cache = nullptr;
  std::vector<int32_t> initial_order;        // free_order as given
  std::vector<int32_t> free_stack;           // back() is handed out next
  std::vector<int32_t> rc;                   // reference count per block
  std::map<int32_t, pkv_seq_state> seqs;     // ordered by id
  int32_t next_id = 0;
  std::vector<std::pair<int32_t, int32_t>> cow_pending;  // (src, dst)
  int64_t alloc_failures = 0;
  int64_t cow_copies = 0;
  int64_t forks = 0;
};

namespace pkv {

// Record a message for pkv_last_error() and return the status.
pkv_status fail(pkv_status st, const std::string& msg);
pkv_status ok();

inline int dtype_bytes(int32_t dt) { return dt == PKV_F32 ? 4 : 2; }

}  // namespace pkv
