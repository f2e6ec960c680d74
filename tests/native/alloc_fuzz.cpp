// Seeded random operations on the host allocator, checking after every call
// the properties of a paged pool: free blocks are distinct and exactly the
// blocks with refcount 0; a refcount equals the number of live tables
// holding the block; a table holds ceil(length / block) blocks; tail waste is
// below one block; a failed call changes nothing.  Built with address and
// undefined-behaviour sanitizers by the CPU test suite.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pkv.h"

#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c);       \
      std::exit(1);                                                           \
    }                                                                         \
  } while (0)

struct Snapshot {
  std::vector<int32_t> free_list, rc, live;
  std::vector<std::vector<int32_t>> tables;
  std::vector<int32_t> lens;
  bool operator==(const Snapshot& o) const {
    return free_list == o.free_list && rc == o.rc && live == o.live && tables == o.tables &&
           lens == o.lens;
  }
};

static Snapshot snap(pkv_pool* p, const pkv_pool_desc& d) {
  Snapshot s;
  int32_t n = 0;
  s.free_list.resize(d.num_blocks + 1);
  CHECK(pkv_free_list(p, s.free_list.data(), d.num_blocks + 1, &n) == PKV_OK);
  s.free_list.resize(n);
  s.rc.resize(d.num_blocks);
  CHECK(pkv_refcounts(p, s.rc.data()) == PKV_OK);
  s.live.resize(4096);
  CHECK(pkv_live_seqs(p, s.live.data(), 4096, &n) == PKV_OK);
  s.live.resize(n);
  for (int32_t id : s.live) {
    std::vector<int32_t> t(d.max_blocks_per_seq);
    int32_t m = 0, len = 0;
    CHECK(pkv_seq_table(p, id, t.data(), d.max_blocks_per_seq, &m) == PKV_OK);
    t.resize(m);
    CHECK(pkv_seq_length(p, id, &len) == PKV_OK);
    s.tables.push_back(t);
    s.lens.push_back(len);
  }
  return s;
}

static void check_invariants(const Snapshot& s, const pkv_pool_desc& d) {
  std::vector<int32_t> holders(d.num_blocks, 0), in_free(d.num_blocks, 0);
  for (int32_t b : s.free_list) {
    CHECK(b >= 0 && b < d.num_blocks);
    CHECK(in_free[b] == 0);
    in_free[b] = 1;
  }
  for (size_t i = 0; i < s.tables.size(); ++i) {
    const auto& t = s.tables[i];
    int64_t need = (int64_t(s.lens[i]) + d.block_size - 1) / d.block_size;
    CHECK(int64_t(t.size()) == need);
    int64_t waste = int64_t(d.block_size) * int64_t(t.size()) - s.lens[i];
    CHECK(waste >= 0 && waste < d.block_size);
    for (int32_t b : t) holders[b]++;
  }
  for (int32_t b = 0; b < d.num_blocks; ++b) {
    CHECK(holders[b] == s.rc[b]);
    CHECK((s.rc[b] == 0) == (in_free[b] == 1));
  }
}

int main(int argc, char** argv) {
  const int seeds = argc > 1 ? std::atoi(argv[1]) : 20;
  for (int seed = 0; seed < seeds; ++seed) {
    std::mt19937 rng(seed);
    pkv_pool_desc d{};
    d.num_blocks = 8 + int(rng() % 56);
    d.block_size = 1 + int(rng() % 16);
    d.num_kv_heads = 1;
    d.head_dim = 64;
    d.max_blocks_per_seq = 1 + int(rng() % 12);
    d.dtype = PKV_F16;
    std::vector<int32_t> order(d.num_blocks);
    for (int32_t i = 0; i < d.num_blocks; ++i) order[i] = i;
    std::shuffle(order.begin(), order.end(), rng);
    pkv_pool* p = nullptr;
    CHECK(pkv_pool_create(&d, nullptr, nullptr, order.data(), &p) == PKV_OK);
    std::vector<int64_t> slots(4096);
    std::vector<int32_t> pairs(2 * 4096);
    for (int op = 0; op < 2000; ++op) {
      Snapshot before = snap(p, d);
      pkv_status st = PKV_OK;
      int kind = int(rng() % 7);
      int32_t any = before.live.empty() ? 12345 : before.live[rng() % before.live.size()];
      if (rng() % 50 == 0) any = 99999;  // unknown id
      int32_t out = 0;
      switch (kind) {
        case 0: st = pkv_seq_alloc(p, int32_t(rng() % (3 * d.block_size * 3)), &out, slots.data()); break;
        case 1: st = pkv_seq_append(p, any, int32_t(rng() % (2 * d.block_size + 2)), slots.data()); break;
        case 2: {
          std::vector<int32_t> b;
          for (int32_t id : before.live)
            if (rng() % 2) b.push_back(id);
          if (rng() % 10 == 0 && !b.empty()) b.push_back(b[0]);  // duplicate -> refused
          st = pkv_seq_append_batch(p, b.data(), int32_t(b.size()), 1 + int32_t(rng() % 2), slots.data());
          if (!b.empty() && b.size() >= 2 && b.back() == b[0]) CHECK(st == PKV_E_BAD_ARG);
          break;
        }
        case 3: st = pkv_seq_fork(p, any, &out); break;
        case 4: st = pkv_seq_free(p, any); break;
        case 5: st = pkv_take_cow(p, pairs.data(), 4096, &out); break;
        case 6: {
          std::vector<int32_t> tab(before.live.size() * d.max_blocks_per_seq + 1), lens(before.live.size() + 1);
          st = pkv_build_batch(p, before.live.data(), int32_t(before.live.size()), tab.data(),
                               d.max_blocks_per_seq, lens.data());
          CHECK(st == PKV_OK);
          break;
        }
      }
      Snapshot after = snap(p, d);
      if (st != PKV_OK) CHECK(after == before);  // all or nothing
      check_invariants(after, d);
    }
    pkv_stats_t s{};
    CHECK(pkv_stats(p, &s) == PKV_OK);
    CHECK(s.free_blocks + s.used_blocks == d.num_blocks);
    CHECK(pkv_pool_destroy(p) == PKV_OK);
  }
  std::printf("alloc_fuzz ok (%d seeds)\n", seeds);
  return 0;
}
