// Shared-block decode plan (host, CPU only).
//
// Sequences forked from one prompt hold the same physical blocks at the same
// table positions ("PagedAttention e continuous batching", 01 · Conceito,
// paragraph 6: requests with an identical prompt prefix point at the same
// read-only blocks).  A decode that walks every table separately reads such
// a block once per holder.  This plan groups the holders: sequences whose
// tables agree on a run of full blocks form a node, and one workgroup per
// (chunk of the node's blocks, set of 128 / group members, KV head) reads the
// chunk once and serves all those members' query heads.  Nodes nest like a
// prefix tree (forks share a prefix of the table), so the batch is walked
// once, depth first: at each depth the sequences still together are split
// by the block they hold there.
#include <algorithm>
#include <cstdlib>
#include <vector>

#include "pool_internal.h"

using pkv::fail;

namespace {

constexpr int32_t kNodeInts = 9;
constexpr int32_t kColumnsPerItem = 128;  // query columns of one wide workgroup
constexpr int32_t kNarrowColumns = 16;    // a node of at most this many columns is narrow
// Chunk sizes without an explicit chunk_tokens: at least kWideChunkBlocks
// (wide) or kNarrowChunkBlocks (narrow), and long nodes cut into at most
// kWideChunks or kNarrowChunks chunks, which keeps the records a sequence
// owns per node few.  The wide launch runs beside the narrow one, which
// hides its length; fewer, longer wide chunks leave fewer records to merge
// and more room on the CUs for narrow workgroups (a 256-sequence batch over
// a 4096-token prefix: 32-block chunks 0.2241-0.2249 ms per decode, 48-block
// 0.2204-0.2208, 64-block 0.2181-0.2187, 128-block 0.2186-0.2201; before
// the two launches overlapped, 32-block chunks were the fastest).
constexpr int32_t kWideChunkBlocks = 64, kNarrowChunkBlocks = 64;
constexpr int32_t kWideChunks = 8, kNarrowChunks = 4;

struct Node {
  int32_t rep, j0, j1, first, members, k_base, first_item, colsets, chunk;
  bool narrow;
};

struct Builder {
  const std::vector<const int32_t*>& rows;  // table of each batch entry
  const std::vector<int32_t>& elig;         // blocks eligible for sharing (all but the last)
  std::vector<int32_t>& priv_start;
  std::vector<int32_t>& n_shared;
  std::vector<int32_t>& order;
  std::vector<Node>& nodes;
  std::vector<int32_t>& buf;  // batch indices being grouped; ranges of it are groups
  int32_t fixed_chunk = 0;    // blocks per chunk when the caller fixed it, else 0
  int32_t per_set = 1;
  int32_t gq = 1;             // query heads per KV head: columns per member
  size_t max_nodes = 0;
  int32_t max_records = 0;    // shared records a sequence may own

  void leaf(int32_t s, int32_t j, int32_t k) {
    priv_start[s] = j;
    n_shared[s] = k;
    order.push_back(s);
  }

  // buf[lo, hi) agree on table entries [0, j0) and each has elig > j0: sort
  // them by the block at j0 and extend every run of two or more into a node
  void split(size_t lo, size_t hi, int32_t j0, int32_t k) {
    std::sort(buf.begin() + lo, buf.begin() + hi, [&](int32_t a, int32_t b) {
      return rows[a][j0] != rows[b][j0] ? rows[a][j0] < rows[b][j0] : a < b;
    });
    size_t i = lo;
    while (i < hi) {
      size_t e = i + 1;
      while (e < hi && rows[buf[e]][j0] == rows[buf[i]][j0]) ++e;
      if (e - i == 1 || nodes.size() >= max_nodes || k >= max_records) {
        for (size_t t = i; t < e; ++t) leaf(buf[t], j0, k);
      } else {
        extend(i, e, j0, k);
      }
      i = e;
    }
  }

  // buf[lo, hi) agree on [0, j0 + 1): take the longest run [j0, j1) all of
  // them hold (one contiguous comparison per member against the first),
  // then continue with those that go on
  void extend(size_t lo, size_t hi, int32_t j0, int32_t k) {
    int32_t j1 = elig[buf[lo]];
    for (size_t t = lo; t < hi; ++t) j1 = std::min(j1, elig[buf[t]]);
    const int32_t* rep = rows[buf[lo]];
    for (size_t t = lo + 1; t < hi && j1 > j0 + 1; ++t)
      j1 = int32_t(std::mismatch(rep + j0 + 1, rep + j1, rows[buf[t]] + j0 + 1).first - rep);
    // narrow nodes (few columns) go to the streaming kernel
    const int32_t members = int32_t(hi - lo);
    const bool narrow = int64_t(members) * gq <= kNarrowColumns;
    int32_t cv = fixed_chunk;
    if (cv == 0) {
      const int32_t parts = narrow ? kNarrowChunks : kWideChunks;
      cv = std::max(narrow ? kNarrowChunkBlocks : kWideChunkBlocks, (j1 - j0 + parts - 1) / parts);
    } else if (narrow) {
      cv = std::max(cv, kNarrowChunkBlocks);
    }
    // a sequence's shared records are capped (the workspace bound counts
    // on it): a node that would pass the cap stops early and its members
    // read the rest of the run as their own blocks
    j1 = int32_t(std::min<int64_t>(j1, j0 + int64_t(max_records - k) * cv));
    const int32_t chunks = (j1 - j0 + cv - 1) / cv;
    Node v;
    v.narrow = narrow;
    v.rep = buf[lo];
    v.j0 = j0;
    v.j1 = j1;
    v.first = int32_t(order.size());
    v.members = members;
    v.k_base = k;
    v.first_item = 0;
    v.colsets = narrow ? 1 : (members + per_set - 1) / per_set;
    v.chunk = cv;
    nodes.push_back(v);
    // members whose sharing ends at j1 first (their own blocks start there),
    // then the rest
    const size_t mid = size_t(std::partition(buf.begin() + lo, buf.begin() + hi,
                                             [&](int32_t s) { return elig[s] == j1; }) -
                              buf.begin());
    for (size_t t = lo; t < mid; ++t) leaf(buf[t], j1, k + chunks);
    if (hi - mid == 1) leaf(buf[mid], j1, k + chunks);
    else if (hi - mid > 1) split(mid, hi, j1, k + chunks);
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
  thread_local std::vector<int32_t> lens, elig, priv_start, n_shared, order, buf;
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

  // PKV_SHARED_CHUNK_TOKENS (read at every call, a multiple of the block
  // size) fixes the chunk size for tuning sweeps when chunk_tokens is 0
  if (chunk_tokens == 0) {
    const char* e = std::getenv("PKV_SHARED_CHUNK_TOKENS");
    const int v = e ? std::atoi(e) : 0;
    if (v > 0 && v % bs == 0) chunk_tokens = v;
  }
  // the prefix tree of the batch, depth first
  priv_start.assign(size_t(n), 0);
  n_shared.assign(size_t(n), 0);
  order.clear();
  nodes.clear();
  Builder b{rows, elig, priv_start, n_shared, order, nodes, buf};
  b.per_set = kColumnsPerItem / group;
  b.gq = group;
  b.max_nodes = size_t(2) * size_t(n);
  b.max_records = PKV_MAX_SHARED_RECORDS;
  b.fixed_chunk = chunk_tokens / bs;
  order.reserve(size_t(n));
  nodes.reserve(b.max_nodes);
  buf.clear();
  for (int32_t i = 0; i < n; ++i)
    if (elig[i] > 0) buf.push_back(i);
  if (buf.size() > 1) b.split(0, buf.size(), 0, 0);
  else for (int32_t s : buf) b.leaf(s, 0, 0);
  for (int32_t i = 0; i < n; ++i)
    if (elig[i] <= 0) order.push_back(i);
  int64_t shared_tokens = 0;
  for (const Node& v : nodes) shared_tokens += int64_t(v.j1 - v.j0) * bs * v.members;
  // the quarter rule of the load-policy hint: below it, the separate launch
  // and the extra records are not worth their cost
  const bool share = total_tokens > 0 && 4 * shared_tokens >= total_tokens;
  if (!share || !eligible) {
    if (pkv_status st = fill_private_plan(lens.data(), n, bs, P, nullptr, nullptr, plan, cap, info)) return st;
    info->shared_kv = share ? 1 : 0;
    return PKV_OK;
  }

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
  // wide nodes first, then narrow ones; each kind numbers its items from 0
  int32_t* nv = sec + 3 * int64_t(n);
  int64_t items[2] = {0, 0};
  int32_t written = 0, n_wide = 0;
  for (int kind = 0; kind < 2; ++kind) {
    for (const Node& v : nodes) {
      if (v.narrow != (kind == 1)) continue;
      const int32_t chunks = (v.j1 - v.j0 + v.chunk - 1) / v.chunk;
      const int32_t w[kNodeInts] = {v.rep,     v.j0,    v.j1, v.first, v.members, v.k_base, int32_t(items[kind]),
                                    v.colsets, v.chunk};
      std::copy(w, w + kNodeInts, nv + kNodeInts * int64_t(written++));
      items[kind] += int64_t(chunks) * v.colsets;
      if (kind == 0) n_wide++;
    }
  }
  if (std::max(items[0], items[1]) * d.num_kv_heads > INT32_MAX)
    return fail(PKV_E_BAD_ARG, "shared plan too large for one launch");
  info->plan_ints = int32_t(need);
  info->n_nodes = int32_t(nodes.size());
  info->n_wide_nodes = n_wide;
  info->n_shared_items = int32_t(items[0]);
  info->n_narrow_items = int32_t(items[1]);
  info->shared_chunk_blocks = b.fixed_chunk > 0 ? b.fixed_chunk : kWideChunkBlocks;
  info->narrow_chunk_blocks = std::max(b.fixed_chunk, kNarrowChunkBlocks);
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
