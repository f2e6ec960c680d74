// Seeded random operations on the host allocator, checking after every call
// the properties of a paged pool: free blocks are distinct and exactly the
// blocks with refcount 0; a refcount equals the number of live tables
// holding the block; a table holds ceil(length / block) blocks; tail waste is
// below one block; a failed call changes nothing.  Then, per seed, the
// hybrid manager, a whole scheduler run and the plan helpers on random
// inputs.  Built with address and undefined-behaviour sanitizers by the CPU
// test suite.
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

// Hybrid manager: slots held == sequences held, refusals change nothing.
static void fuzz_hybrid(std::mt19937& rng) {
  pkv_pool_desc d{};
  d.num_blocks = 4 + int(rng() % 40);
  d.block_size = 16;
  d.num_kv_heads = 1;
  d.head_dim = 8;
  d.max_blocks_per_seq = 1 + int(rng() % 8);
  d.dtype = PKV_BF16;
  pkv_pool* p = nullptr;
  CHECK(pkv_pool_create(&d, nullptr, nullptr, nullptr, &p) == PKV_OK);
  const int32_t ns = 1 + int32_t(rng() % 10);
  pkv_hybrid* h = nullptr;
  CHECK(pkv_hybrid_create(p, ns, 64, nullptr, nullptr, &h) == PKV_OK);
  std::vector<int32_t> held;
  std::vector<int32_t> pairs(2 * 1024);
  for (int op = 0; op < 500; ++op) {
    pkv_hybrid_stats_t a{}, b{};
    CHECK(pkv_hybrid_stats(h, &a) == PKV_OK);
    const int kind = int(rng() % 4);
    int32_t seq = -1, slot = -1, n = 0;
    pkv_status st = PKV_OK;
    if (kind == 0) {
      st = pkv_hybrid_admit(h, int32_t(rng() % 80), &seq, &slot, nullptr);
      if (st == PKV_OK) held.push_back(seq);
    } else if (kind == 1 && !held.empty()) {
      st = pkv_hybrid_fork(h, held[rng() % held.size()], &seq, &slot);
      if (st == PKV_OK) held.push_back(seq);
    } else if (kind == 2 && !held.empty()) {
      const size_t i = rng() % held.size();
      CHECK(pkv_hybrid_free(h, held[i]) == PKV_OK);
      held.erase(held.begin() + i);
    } else {
      CHECK(pkv_hybrid_take_copies(h, pairs.data(), 1024, &n) == PKV_OK);
      for (int32_t i = 0; i < 2 * n; ++i) CHECK(pairs[i] >= 0 && pairs[i] < ns);
    }
    CHECK(pkv_hybrid_stats(h, &b) == PKV_OK);
    CHECK(b.free_slots + b.used_slots == ns);
    CHECK(b.used_slots == int64_t(held.size()));
    if (st != PKV_OK) CHECK(b.used_slots == a.used_slots && b.refusals >= a.refusals);
  }
  for (int32_t s : held) CHECK(pkv_hybrid_free(h, s) == PKV_OK);
  pkv_stats_t ps{};
  CHECK(pkv_stats(p, &ps) == PKV_OK);
  CHECK(ps.used_blocks == 0);
  CHECK(pkv_hybrid_destroy(h) == PKV_OK);
  CHECK(pkv_pool_destroy(p) == PKV_OK);
}

// Scheduler: runs a random request stream to the end; every request ends
// finished with all its tokens or rejected, and the pool ends empty.
static void fuzz_scheduler(std::mt19937& rng) {
  pkv_pool_desc d{};
  d.num_blocks = 16 + int(rng() % 200);
  d.block_size = 16;
  d.num_kv_heads = 1;
  d.head_dim = 8;
  d.max_blocks_per_seq = 4 + int(rng() % 40);
  d.dtype = PKV_F16;
  pkv_pool* p = nullptr;
  CHECK(pkv_pool_create(&d, nullptr, nullptr, nullptr, &p) == PKV_OK);
  const int32_t n = 1 + int32_t(rng() % 40);
  std::vector<pkv_request> reqs(n);
  for (int32_t i = 0; i < n; ++i) {
    pkv_request& r = reqs[i];
    r.arrival = int32_t(rng() % 50);
    r.prompt_len = 1 + int32_t(rng() % 400);
    r.output_len = 1 + int32_t(rng() % 60);
    r.klass = int32_t(rng() % 2);
    r.prefix_id = rng() % 3 == 0 ? int32_t(rng() % 2) : -1;
    r.prefix_len = r.prefix_id >= 0 ? 16 * int32_t(rng() % 4) : 0;
    if (r.prefix_id >= 0 && r.prompt_len <= r.prefix_len) r.prompt_len = r.prefix_len + 1;
  }
  pkv_sched_config cfg{};
  cfg.max_batch_tokens = 8 + int32_t(rng() % 512);
  cfg.chunk_tokens = 1 + int32_t(rng() % 256);
  cfg.max_running = 1 + int32_t(rng() % 16);
  pkv_sched* s = nullptr;
  CHECK(pkv_sched_create(p, &cfg, reqs.data(), n, &s) == PKV_OK);
  std::vector<pkv_sched_item> items(cfg.max_running);
  pkv_sched_stats_t st{};
  int steps = 0;
  do {
    pkv_sched_step_info info{};
    CHECK(pkv_sched_step(s, items.data(), cfg.max_running, &info) == PKV_OK);
    CHECK(info.n_items <= cfg.max_running);
    CHECK(info.prefill_tokens + info.decode_tokens <= cfg.max_batch_tokens);
    CHECK(pkv_sched_stats(s, &st) == PKV_OK);
    CHECK(++steps < 200000);
  } while (st.finished + st.rejected < n);
  pkv_sched_step_info info{};
  CHECK(pkv_sched_step(s, items.data(), cfg.max_running, &info) == PKV_OK && info.n_items == 0);
  for (int32_t i = 0; i < n; ++i) {
    pkv_request_state rs{};
    CHECK(pkv_sched_request(s, i, &rs) == PKV_OK);
    CHECK(rs.state == PKV_REQ_REJECTED || (rs.state == PKV_REQ_FINISHED && rs.generated == reqs[i].output_len));
  }
  pkv_stats_t ps{};
  CHECK(pkv_stats(p, &ps) == PKV_OK);
  CHECK(ps.used_blocks == 0 && ps.free_blocks == d.num_blocks);
  CHECK(pkv_sched_destroy(s) == PKV_OK);
  CHECK(pkv_pool_destroy(p) == PKV_OK);
}

// Plans and the utilisation count on random inputs (bounds of the outputs).
static void fuzz_plans(std::mt19937& rng) {
  const int32_t b = 1 + int32_t(rng() % 20);
  std::vector<int32_t> ql(b), cl(b);
  for (int32_t i = 0; i < b; ++i) {
    ql[i] = 1 + int32_t(rng() % 300);
    cl[i] = ql[i] + int32_t(rng() % 2000);
  }
  const int32_t hkv = 1 + int32_t(rng() % 4), hq = hkv * (1 + int32_t(rng() % 20));
  const int32_t max_keys = rng() % 2 ? 0 : 32 * (1 + int32_t(rng() % 40));
  int32_t need = 0;
  CHECK(pkv_prefill_plan_ints(ql.data(), cl.data(), b, hq, hkv, max_keys, &need) == PKV_OK);
  std::vector<int32_t> plan(need);
  pkv_prefill_plan_info info{};
  CHECK(pkv_prefill_plan(ql.data(), cl.data(), b, hq, hkv, max_keys, plan.data(), need, &info) == PKV_OK);
  CHECK(info.plan_ints == need);
  for (int32_t w = 0; w < info.n_work; ++w) {
    const int32_t* e = plan.data() + 6 * w;
    CHECK(e[0] >= 0 && e[0] < b);
    CHECK(e[1] >= 0 && e[1] * info.tile_tokens < ql[e[0]]);
    CHECK(0 <= e[2] && e[2] < e[3]);
    CHECK(e[4] < info.n_split && e[5] >= 0);
  }
  CHECK(pkv_prefill_plan(ql.data(), cl.data(), b, hq, hkv, max_keys, plan.data(), need - 1, &info) ==
        PKV_E_BAD_ARG);
  pkv_utilisation_t u{};
  CHECK(pkv_utilisation(ql.data(), b, 300, 16, &u) == PKV_OK);
  CHECK(u.paged_waste_tokens >= 0 && u.paged_waste_tokens < 16 * b);
}

// Shared-block plans over forked batches: every block of every sequence is
// covered exactly once (by the chunks of the nodes it belongs to, or by its
// own range), node members hold the node's blocks at the same positions and
// never their last block, record indices are distinct and capped, and the
// order array keeps each node's members contiguous.
static void fuzz_shared_plan(std::mt19937& rng) {
  pkv_pool_desc d{};
  d.num_blocks = 400;
  d.block_size = 16;
  d.num_kv_heads = 1 << int(rng() % 3);
  d.head_dim = 128;
  d.max_blocks_per_seq = 40;
  d.dtype = PKV_F16;
  pkv_pool* p = nullptr;
  CHECK(pkv_pool_create(&d, nullptr, nullptr, nullptr, &p) == PKV_OK);
  std::vector<int32_t> live;
  int32_t s0 = 0;
  CHECK(pkv_seq_alloc(p, 16 * int32_t(1 + rng() % 12), &s0, nullptr) == PKV_OK);
  live.push_back(s0);
  for (int op = 0; op < 60; ++op) {
    const int32_t any = live[rng() % live.size()];
    int32_t out = 0, len = 0;
    CHECK(pkv_seq_length(p, any, &len) == PKV_OK);
    const int kind = int(rng() % 3);
    if (kind == 0 && pkv_seq_fork(p, any, &out) == PKV_OK) live.push_back(out);
    if (kind == 1 && pkv_seq_fork_prefix(p, any, int32_t(rng() % (len + 1)), &out) == PKV_OK) live.push_back(out);
    if (kind == 2) (void)pkv_seq_append(p, any, 1 + int32_t(rng() % 40), nullptr);
  }
  std::vector<int32_t> seqs;
  for (int32_t id : live) {
    int32_t len = 0;
    CHECK(pkv_seq_length(p, id, &len) == PKV_OK);
    if (len > 0 && rng() % 8 != 0) seqs.push_back(id);
  }
  const int32_t n = int32_t(seqs.size());
  const int32_t groups[] = {1, 2, 4, 8, 16};
  const int32_t group = groups[rng() % 5];
  const int32_t chunks[] = {0, 16, 64, 256};
  const int32_t chunk_tokens = chunks[rng() % 4];
  const int32_t P = 16 * int32_t(1 + rng() % 8);
  int32_t need = 0;
  CHECK(pkv_decode_plan_shared_ints(p, seqs.data(), n, P, &need) == PKV_OK);
  std::vector<int32_t> plan(size_t(need) + 1);
  pkv_decode_plan_info info{};
  CHECK(pkv_decode_plan_shared(p, seqs.data(), n, P, group * d.num_kv_heads, chunk_tokens, plan.data(), need,
                               &info) == PKV_OK);
  CHECK(info.plan_ints <= need);
  std::vector<std::vector<int32_t>> tab(n);
  std::vector<int32_t> nblk(n), cover_count;
  for (int32_t i = 0; i < n; ++i) {
    tab[i].resize(d.max_blocks_per_seq);
    int32_t m = 0, len = 0;
    CHECK(pkv_seq_table(p, seqs[i], tab[i].data(), d.max_blocks_per_seq, &m) == PKV_OK);
    CHECK(pkv_seq_length(p, seqs[i], &len) == PKV_OK);
    nblk[i] = (len + 15) / 16;
    CHECK(m == nblk[i]);
  }
  std::vector<std::vector<int32_t>> cover(n);
  for (int32_t i = 0; i < n; ++i) cover[i].assign(nblk[i], 0);
  const int32_t* part_offset = plan.data() + 2 * info.n_work;
  const int32_t pb = P / 16;
  std::vector<int32_t> priv(n, 0), nsh(n, 0);
  if (info.n_nodes > 0) {
    const int32_t* sec = plan.data() + info.off_shared;
    const int32_t* order = sec + 2 * n;
    const int32_t* nodes = sec + 3 * n;
    std::vector<int32_t> seen(n, 0);
    for (int32_t i = 0; i < n; ++i) {
      priv[i] = sec[i];
      nsh[i] = sec[n + i];
      CHECK(order[i] >= 0 && order[i] < n && !seen[order[i]]);
      seen[order[i]] = 1;
      CHECK(nsh[i] <= PKV_MAX_SHARED_RECORDS);
    }
    std::vector<std::vector<int32_t>> recs(n);
    int64_t items[2] = {0, 0};
    for (int32_t v = 0; v < info.n_nodes; ++v) {
      const int32_t* nd = nodes + 9 * v;
      const int32_t rep = nd[0], j0 = nd[1], j1 = nd[2], first = nd[3], mem = nd[4], kb = nd[5];
      const int narrow = v >= info.n_wide_nodes ? 1 : 0;
      CHECK((mem * group <= 16) == (narrow == 1));
      const int32_t cb = nd[8];
      CHECK(cb >= (narrow ? info.narrow_chunk_blocks : info.shared_chunk_blocks));
      CHECK(nd[6] == items[narrow] && j0 < j1 && mem >= 2 && first + mem <= n);
      CHECK(nd[7] == (narrow ? 1 : (mem * group + 127) / 128));
      const int32_t nch = (j1 - j0 + cb - 1) / cb;
      items[narrow] += int64_t(nch) * nd[7];
      bool rep_in = false;
      for (int32_t t = first; t < first + mem; ++t) {
        const int32_t s = order[t];
        rep_in |= (s == rep);
        CHECK(j1 <= nblk[s] - 1);
        for (int32_t j = j0; j < j1; ++j) {
          CHECK(tab[s][j] == tab[rep][j]);
          cover[s][j]++;
        }
        for (int32_t c = 0; c < nch; ++c) recs[s].push_back(kb + c);
      }
      CHECK(rep_in);
    }
    CHECK(items[0] == info.n_shared_items && items[1] == info.n_narrow_items);
    for (int32_t i = 0; i < n; ++i) {
      std::sort(recs[i].begin(), recs[i].end());
      CHECK(int32_t(recs[i].size()) == nsh[i]);
      for (int32_t r = 0; r < nsh[i]; ++r) CHECK(recs[i][r] == r);
    }
  }
  // private ranges through the work items
  int32_t partials = 0;
  std::vector<int32_t> parts_seen(n, 0);
  for (int32_t w = 0; w < info.n_work; ++w) {
    const int32_t s = plan[2 * w], q = plan[2 * w + 1];
    CHECK(s >= 0 && s < n);
    const int32_t b0 = priv[s] + q * pb, b1 = std::min(b0 + pb, nblk[s]);
    CHECK(b0 < b1);
    for (int32_t j = b0; j < b1; ++j) cover[s][j]++;
    parts_seen[s]++;
  }
  for (int32_t i = 0; i < n; ++i) {
    for (int32_t j = 0; j < nblk[i]; ++j) CHECK(cover[i][j] == 1);
    const int32_t records = nsh[i] + parts_seen[i];
    if (records > 1) {
      CHECK(part_offset[i] == partials);
      partials += records;
    } else {
      CHECK(part_offset[i] == -1);
    }
  }
  CHECK(partials == info.n_partials);
  CHECK(pkv_pool_destroy(p) == PKV_OK);
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
      int kind = int(rng() % 8);
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
        case 7: {
          int32_t len = 0;
          const bool known = pkv_seq_length(p, any, &len) == PKV_OK;
          const int32_t n = known ? int32_t(rng() % (len + 2)) : 3;  // len + 1: refused
          st = pkv_seq_fork_prefix(p, any, n, &out);
          if (known && n > len) CHECK(st == PKV_E_BAD_ARG);
          break;
        }
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
    fuzz_hybrid(rng);
    fuzz_scheduler(rng);
    fuzz_plans(rng);
    for (int k = 0; k < 4; ++k) fuzz_shared_plan(rng);
  }
  std::printf("alloc_fuzz ok (%d seeds)\n", seeds);
  return 0;
}
