// Internal state of a pkv_hybrid (shared by the host manager and the device
// copy entry point).  Plain C++17.
#pragma once

#include <cstdint>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pool_internal.h"

struct pkv_hybrid {
  pkv_pool* kv = nullptr;
  int32_t num_slots = 0;
  int64_t slot_bytes = 0;
  void* state_base = nullptr;                 // device, num_slots * slot_bytes, or null
  std::vector<int32_t> free_slots;            // back() is handed out next
  std::unordered_map<int32_t, int32_t> slot_of;  // live sequence -> state slot
  std::vector<std::pair<int32_t, int32_t>> copies;  // queued (src, dst) state copies
  int64_t refusals = 0;
  int64_t state_copies = 0;
};
