// Shared-block decode plan (host, CPU only).
//
// Sequences forked from one prompt hold the same physical blocks at the same
// table positions ("PagedAttention e continuous batching", 01 · Conceito,
// paragraph 6: requests with an identical prompt prefix point at the same
// read-only blocks).  A decode that walks every table separately reads such
// a block once per holder.  This plan groups the holders: sequences whose
// tables agree on a run of full blocks form a node, and one workgroup per
// (chunk of the node's blocks, set of 64 / group members, KV head) reads the
// chunk once and serves all those members' query heads.  Nodes nest like a
// prefix tree (forks share a prefix of the table), so the batch is walked
// once, depth first: at each depth the sequences still together are split
// by the block they hold there.
#include <algorithm>
#include <vector>

#include "pool_internal.h"

using pkv::fail;

namespace {

constexpr int32_t kNodeInts = 8;
constexpr int32_t kColumnsPerItem = 64;     // query columns of one shared workgroup
constexpr int64_t kTargetSharedWorkgroups = 512;
constexpr int32_t kMinChunkBlocks = 16, kMaxChunkBlocks = 256;

struct Node {
  int32_t rep, j0, j1, first, members, k_base, first_item, colsets;
};

struct Builder {
  const std::vector<const int32_t*>& rows;  // table of each batch entry
  const std::vector<int32_t>& elig;         // blocks eligible for sharing (all but the last)
  std::vector<int32_t>& priv_start;
  std::vector<int32_t>& n_shared;
  std::vector<int32_t>& order;
  std::vector<Node>& nodes;
  int32_t chunk = 0;  // blocks per chunk; 0 while only the tree is built
  int32_t per_set = 1;
  size_t max_nodes = 0;
  int32_t max_records = 0;  // shared records a sequence may own (with chunk > 0)

  void leaf(int32_t s, int32_t j, int32_t k) {
    priv_start[s] = j;
    n_shared[s] = k;
    order.push_back(s);
  }

  // members agree on table entries [0, j0) and each has elig > j0; split them
  // by the block at j0 and extend every group of two or more into a node
  void split(std::vector<int32_t> members, int32_t j0, int32_t k) {
    std::sort(members.begin(), members.end(), [&](int32_t a, int32_t b) {
      return rows[a][j0] != rows[b][j0] ? rows[a][j0] < rows[b][j0] : a < b;
    });
    size_t i = 0;
    while (i < members.size()) {
      size_t e = i + 1;
      while (e < members.size() && rows[members[e]][j0] == rows[members[i]][j0]) ++e;
      if (e - i == 1 || nodes.size() >= max_nodes || (chunk > 0 && k >= max_records)) {
        for (size_t t = i; t < e; ++t) leaf(members[t], j0, k);
      } else {
        extend(std::vector<int32_t>(members.begin() + i, members.begin() + e), j0, k);
      }
      i = e;
    }
  }

  // the group agrees on [0, j0 + 1): take the longest run [j0, j1) all of
  // its members hold, then continue with those that go on
  void extend(std::vector<int32_t> group, int32_t j0, int32_t k) {
    int32_t emin = elig[group[0]];
    for (int32_t s : group) emin = std::min(emin, elig[s]);
    const int32_t* rep = rows[group[0]];
    int32_t j1 = j0 + 1;
    while (j1 < emin) {
      bool same = true;
      for (int32_t s : group)
        if (rows[s][j1] != rep[j1]) {
          same = false;
          break;
        }
      if (!same) break;
      ++j1;
    }
    // a sequence's shared records are capped (the workspace bound counts
    // on it): a node that would pass the cap stops early and its members
    // read the rest of the run as their own blocks
    if (chunk > 0) j1 = std::min<int64_t>(j1, j0 + int64_t(max_records - k) * chunk);
    const int32_t chunks = chunk > 0 ? (j1 - j0 + chunk - 1) / chunk : 1;
    Node v;
    v.rep = group[0];
    v.j0 = j0;
    v.j1 = j1;
    v.first = int32_t(order.size());
    v.members = int32_t(group.size());
    v.k_base = k;
    v.first_item = 0;
    v.colsets = (v.members + per_set - 1) / per_set;
    nodes.push_back(v);
    std::vector<int32_t> rest;
    for (int32_t s : group) {
      if (elig[s] == j1) leaf(s, j1, k + chunks);  // its own blocks start here
      else rest.push_back(s);
    }
    if (rest.size() == 1) leaf(rest[0], j1, k + chunks);
    else if (rest.size() > 1) split(std::move(rest), j1, k + chunks);
  }
};

}  // namespace

namespace pkv {

int64_t shared_plan_bound(int64_t n, int64_t total_blocks, int32_t pblocks) {
  // private part: 2 ints per partition (at most one more partition per
  // sequence than its blocks alone need), part offsets, reduce list; shared
  // section: three per-sequence arrays and at most 2n nodes
  return 2 * (total_blocks / pblocks + n) + 2 * n + 3 * n + kNodeInts * 2 * n;
}

pkv_status build_shared_plan(const pkv_pool* p, const int32_t* seqs, int32_t n, int32_t P,
                             int32_t num_q_heads, int32_t chunk_tokens, int32_t* plan, int64_t cap,
                             pkv_decode_plan_info* info) {
  const pkv_pool_desc& d = p->desc;
  const int32_t bs = d.block_size;
  if (P == 0) P = kDefaultPartitionTokens;
  if (P < bs || P % bs != 0)
    return fail(PKV_E_BAD_ARG, "partition_tokens must be a positive multiple of block_size");
  if (chunk_tokens < 0 || chunk_tokens % bs != 0)
    return fail(PKV_E_BAD_ARG, "chunk_tokens must be 0 or a positive multiple of block_size");
  if (num_q_heads < 1 || num_q_heads % d.num_kv_heads != 0)
    return fail(PKV_E_BAD_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  thread_local std::vector<const int32_t*> rows;
  thread_local std::vector<int32_t> lens, elig, priv_start, n_shared, order;
  thread_local std::vector<Node> nodes;
  rows.resize(size_t(n));
  lens.resize(size_t(n));
  elig.resize(size_t(n));
  int64_t total_tokens = 0;
  for (int32_t i = 0; i < n; ++i) {
    const pkv_seq_state* s = find_seq(p, seqs[i]);
    if (!s) return fail(PKV_E_BAD_SEQ, "unknown sequence " + std::to_string(seqs[i]));
    if (s->length < 1) return fail(PKV_E_BAD_ARG, "every context length must be >= 1");
    rows[i] = s->table.data();
    lens[i] = s->length;
    elig[i] = int32_t(s->table.size()) - 1;
    total_tokens += s->length;
  }
  const int32_t group = num_q_heads / d.num_kv_heads;
  const bool eligible = (d.dtype == PKV_F16 || d.dtype == PKV_BF16) && d.head_dim == 128 && bs == 16 &&
                        group <= 16 && 16 % group == 0;

  // the prefix tree of the batch (chunk size not yet known)
  priv_start.assign(size_t(n), 0);
  n_shared.assign(size_t(n), 0);
  order.clear();
  nodes.clear();
  Builder b{rows, elig, priv_start, n_shared, order, nodes};
  b.per_set = kColumnsPerItem / group;
  b.max_nodes = size_t(2) * size_t(n);
  b.max_records = PKV_MAX_SHARED_RECORDS;
  {
    std::vector<int32_t> all;
    for (int32_t i = 0; i < n; ++i)
      if (elig[i] > 0) all.push_back(i);
    if (all.size() > 1) b.split(std::move(all), 0, 0);
    else for (int32_t s : all) b.leaf(s, 0, 0);
  }
  int64_t shared_tokens = 0, units = 0;
  for (const Node& v : nodes) {
    shared_tokens += int64_t(v.j1 - v.j0) * bs * v.members;
    units += int64_t(v.j1 - v.j0) * v.colsets;
  }
  // the quarter rule of the load-policy hint: below it, the separate launch
  // and the extra records are not worth their cost
  const bool share = total_tokens > 0 && 4 * shared_tokens >= total_tokens;
  if (!share || !eligible) {
    if (pkv_status st = fill_private_plan(lens.data(), n, bs, P, nullptr, nullptr, plan, cap, info)) return st;
    info->shared_kv = share ? 1 : 0;
    return PKV_OK;
  }

  // chunk size, then the tree again with record counts per chunk
  int32_t chunk = chunk_tokens / bs;
  if (chunk == 0) {
    const int64_t c = (units * d.num_kv_heads + kTargetSharedWorkgroups - 1) / kTargetSharedWorkgroups;
    chunk = int32_t(std::min<int64_t>(kMaxChunkBlocks, std::max<int64_t>(kMinChunkBlocks, c)));
  }
  priv_start.assign(size_t(n), 0);
  n_shared.assign(size_t(n), 0);
  order.clear();
  nodes.clear();
  b.chunk = chunk;
  {
    std::vector<int32_t> all;
    for (int32_t i = 0; i < n; ++i)
      if (elig[i] > 0) all.push_back(i);
    if (all.size() > 1) b.split(std::move(all), 0, 0);
    else for (int32_t s : all) b.leaf(s, 0, 0);
  }
  for (int32_t i = 0; i < n; ++i)
    if (elig[i] <= 0) order.push_back(i);

  if (pkv_status st = fill_private_plan(lens.data(), n, bs, P, priv_start.data(), n_shared.data(), plan, cap,
                                        info))
    return st;
  const int64_t off = info->plan_ints;
  const int64_t need = off + 3 * int64_t(n) + kNodeInts * int64_t(nodes.size());
  if (need > INT32_MAX || need > cap) return fail(PKV_E_BAD_ARG, "plan buffer too small");
  int32_t* sec = plan + off;
  std::copy(priv_start.begin(), priv_start.end(), sec);
  std::copy(n_shared.begin(), n_shared.end(), sec + n);
  std::copy(order.begin(), order.end(), sec + 2 * int64_t(n));
  int32_t* nv = sec + 3 * int64_t(n);
  int64_t items = 0;
  for (size_t t = 0; t < nodes.size(); ++t) {
    const Node& v = nodes[t];
    const int32_t chunks = (v.j1 - v.j0 + chunk - 1) / chunk;
    const int32_t w[kNodeInts] = {v.rep, v.j0, v.j1, v.first, v.members, v.k_base, int32_t(items), v.colsets};
    std::copy(w, w + kNodeInts, nv + kNodeInts * t);
    items += int64_t(chunks) * v.colsets;
  }
  if (items * d.num_kv_heads > INT32_MAX) return fail(PKV_E_BAD_ARG, "shared plan too large for one launch");
  info->plan_ints = int32_t(need);
  info->n_nodes = int32_t(nodes.size());
  info->n_shared_items = int32_t(items);
  info->shared_chunk_blocks = chunk;
  info->shared_group = group;
  info->off_shared = int32_t(off);
  info->shared_kv = 0;  // what is left per sequence is its own
  return PKV_OK;
}

}  // namespace pkv

extern "C" {

pkv_status pkv_decode_plan_shared_ints(const pkv_pool* pool, const int32_t* seqs, int32_t n_seqs,
                                       int32_t partition_tokens, int32_t* plan_ints) {
  if (!pool || !plan_ints || n_seqs < 0 || (n_seqs > 0 && !seqs))
    return fail(PKV_E_BAD_ARG, "null pool, sequences or output");
  const int32_t P = partition_tokens ? partition_tokens : pkv::kDefaultPartitionTokens;
  const int32_t bs = pool->desc.block_size;
  if (P < bs || P % bs != 0)
    return fail(PKV_E_BAD_ARG, "partition_tokens must be a positive multiple of block_size");
  int64_t blocks = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const pkv_seq_state* s = pkv::find_seq(pool, seqs[i]);
    if (!s) return fail(PKV_E_BAD_SEQ, "unknown sequence " + std::to_string(seqs[i]));
    blocks += int64_t(s->table.size());
  }
  const int64_t b = pkv::shared_plan_bound(n_seqs, blocks, P / bs);
  if (b > INT32_MAX) return fail(PKV_E_BAD_ARG, "plan too large");
  *plan_ints = int32_t(b);
  return PKV_OK;
}

pkv_status pkv_decode_plan_shared(const pkv_pool* pool, const int32_t* seqs, int32_t n_seqs,
                                  int32_t partition_tokens, int32_t num_q_heads, int32_t chunk_tokens,
                                  int32_t* plan, int32_t cap, pkv_decode_plan_info* info) {
  if (!pool || !info || n_seqs < 0 || (n_seqs > 0 && !seqs) || (cap > 0 && !plan))
    return fail(PKV_E_BAD_ARG, "null pool, sequences, plan or info");
  return pkv::build_shared_plan(pool, seqs, n_seqs, partition_tokens, num_q_heads, chunk_tokens, plan, cap, info);
}

}  // extern "C"
