// Host half of one decode iteration in a single call (CPU only): append the
// new tokens, take the copy-on-write pairs, build block tables, lengths and
// the split-K plan, all into one caller-provided staging buffer so that one
// host-to-device copy moves the whole iteration's metadata.
#include <algorithm>

#include "pool_internal.h"

using pkv::fail;

namespace {

constexpr int64_t kAlign = 256;

int64_t align_up(int64_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

struct Offsets {
  int64_t slots, pairs, tables, lens, plan, end;
};

Offsets layout_for(int64_t n, int64_t append, int64_t pair_cap, int64_t stride, int64_t plan_cap) {
  Offsets o;
  o.slots = 0;
  o.pairs = o.slots + align_up(8 * n * append);
  o.tables = o.pairs + align_up(8 * pair_cap);
  o.lens = o.tables + align_up(4 * n * stride);
  o.plan = o.lens + align_up(4 * n);
  o.end = o.plan + align_up(4 * plan_cap);
  return o;
}

// Whether at least a quarter of the batch's context tokens lie in blocks that
// more than one sequence holds (the K/V load policy hint of the decode plan).
// Blocks are shared only through forks ("PagedAttention e continuous
// batching", 01 · Conceito, paragraph 6: sequences with a common prefix point
// at the same read-only blocks, a diverging writer gets a copy): a child takes
// its parent's whole table, and copy-on-write replaces only the partly filled
// last block, so along a table the holders of block j include
// those of block j + 1 and the reference counts never increase: the shared
// blocks are a prefix of the table, found by bisection.  The quarter is the
// break-even point measured on MI355X: streaming (nontemporal) loads read
// unshared tiles ~12% faster, cached loads read a prefix shared by 256
// sequences ~2x faster.
bool shares_context(const pkv_pool* p, const int32_t* seqs, int32_t n) {
  const int32_t bs = p->desc.block_size;
  int64_t total = 0, shared = 0;
  for (int32_t i = 0; i < n; ++i) {
    const pkv_seq_state* s = pkv::find_seq(p, seqs[i]);
    const int32_t nblk = (s->length + bs - 1) / bs;
    int32_t lo = 0, hi = nblk;  // first block with a single holder lies in [lo, hi]
    while (lo < hi) {
      const int32_t mid = lo + (hi - lo) / 2;
      if (p->rc[size_t(s->table[size_t(mid)])] > 1) lo = mid + 1;
      else hi = mid;
    }
    total += s->length;
    shared += std::min<int64_t>(s->length, int64_t(lo) * bs);
  }
  return total > 0 && 4 * shared >= total;
}

int64_t plan_cap_for(int64_t n, int64_t stride, int32_t bs, int32_t P) {
  const int64_t max_parts = (stride * bs + P - 1) / P;
  return std::max(2 * n * max_parts + 2 * n, pkv::shared_plan_bound(n, n * stride, P / bs));
}

}  // namespace

extern "C" {

size_t pkv_prepare_decode_bytes(int32_t max_seqs, int32_t append_tokens, int32_t table_stride,
                                int32_t block_size, int32_t partition_tokens) {
  if (max_seqs < 0 || append_tokens < 0 || table_stride < 1 || block_size < 1) return 0;
  const int32_t P = pkv::sizing_partition(partition_tokens);
  if (P < block_size) return 0;
  const Offsets o = layout_for(max_seqs, append_tokens, max_seqs, table_stride,
                               plan_cap_for(max_seqs, table_stride, block_size, P));
  return size_t(o.end);
}

pkv_status pkv_batch_shared_kv(const pkv_pool* p, const int32_t* seqs, int32_t n_seqs,
                               int32_t* shared_kv) {
  if (!p || !shared_kv || n_seqs < 0 || (n_seqs > 0 && !seqs))
    return fail(PKV_E_BAD_ARG, "null pool, sequences or output");
  for (int32_t i = 0; i < n_seqs; ++i)
    if (!pkv::find_seq(p, seqs[i])) return fail(PKV_E_BAD_SEQ, "unknown sequence " + std::to_string(seqs[i]));
  *shared_kv = shares_context(p, seqs, n_seqs) ? 1 : 0;
  return PKV_OK;
}

pkv_status pkv_prepare_decode(pkv_pool* p, const int32_t* seqs, int32_t n_seqs,
                              int32_t append_tokens, int32_t table_stride,
                              int32_t partition_tokens, int32_t num_q_heads, void* staging,
                              size_t staging_bytes, pkv_batch_layout* layout) {
  if (!p || !layout || !staging) return fail(PKV_E_BAD_ARG, "null pool, staging or layout");
  if (n_seqs < 0 || append_tokens < 0 || table_stride < 1 || (n_seqs > 0 && !seqs))
    return fail(PKV_E_BAD_ARG, "bad batch arguments");
  if (num_q_heads < 0 || (num_q_heads > 0 && num_q_heads % p->desc.num_kv_heads != 0))
    return fail(PKV_E_BAD_ARG, "num_q_heads must be 0 or a positive multiple of num_kv_heads");
  const int32_t bs = p->desc.block_size;
  const int32_t P = partition_tokens ? partition_tokens : pkv::kDefaultPartitionTokens;
  if (P < bs || P % bs != 0)
    return fail(PKV_E_BAD_ARG, "partition_tokens must be a positive multiple of block_size");
  if (reinterpret_cast<uintptr_t>(staging) % 8 != 0)
    return fail(PKV_E_BAD_ARG, "staging buffer must be 8-byte aligned");
  // every check that could fail comes before the pool changes
  for (int32_t i = 0; i < n_seqs; ++i) {
    const pkv_seq_state* s = pkv::find_seq(p, seqs[i]);
    if (!s) return fail(PKV_E_BAD_SEQ, "unknown sequence " + std::to_string(seqs[i]));
    const int64_t after = int64_t(s->length) + append_tokens;
    if (after < 1) return fail(PKV_E_BAD_ARG, "a sequence in the batch has no tokens to attend");
    if ((after + bs - 1) / bs > table_stride)
      return fail(PKV_E_BAD_ARG, "a table would be wider than table_stride");
  }
  const int64_t pair_cap = int64_t(p->cow_pending.size()) + (append_tokens > 0 ? n_seqs : 0);
  const Offsets o = layout_for(n_seqs, append_tokens, pair_cap, table_stride,
                               plan_cap_for(n_seqs, table_stride, bs, P));
  if (int64_t(staging_bytes) < o.end)
    return fail(PKV_E_BAD_ARG, "staging buffer too small: need " + std::to_string(o.end) + " bytes");
  char* base = static_cast<char*>(staging);
  int64_t* slots = reinterpret_cast<int64_t*>(base + o.slots);
  int32_t* pairs = reinterpret_cast<int32_t*>(base + o.pairs);
  int32_t* tables = reinterpret_cast<int32_t*>(base + o.tables);
  int32_t* lens = reinterpret_cast<int32_t*>(base + o.lens);
  int32_t* plan = reinterpret_cast<int32_t*>(base + o.plan);

  if (append_tokens > 0) {
    if (pkv_status st = pkv_seq_append_batch(p, seqs, n_seqs, append_tokens, slots)) return st;
  }
  int32_t n_pairs = 0;
  pkv_take_cow(p, pairs, int32_t(pair_cap), &n_pairs);
  pkv_build_batch(p, seqs, n_seqs, tables, table_stride, lens);
  pkv_decode_plan_info info{};
  const int64_t cap = plan_cap_for(n_seqs, table_stride, bs, P);
  if (num_q_heads > 0) {
    // blocks held in common are read once for all their holders
    if (pkv_status st = pkv::build_shared_plan(p, seqs, n_seqs, P, num_q_heads, 0, plan, cap, &info))
      return st;  // unreachable: ids and lengths were checked above
  } else {
    if (pkv_status st = pkv_decode_plan(lens, n_seqs, bs, P, plan, int32_t(cap), &info))
      return st;  // unreachable: lengths were checked above
    info.shared_kv = shares_context(p, seqs, n_seqs) ? 1 : 0;
  }
  layout->n_seqs = n_seqs;
  layout->append_tokens = append_tokens;
  layout->n_pairs = n_pairs;
  layout->table_stride = table_stride;
  layout->off_slots = o.slots;
  layout->off_pairs = o.pairs;
  layout->off_tables = o.tables;
  layout->off_lens = o.lens;
  layout->off_plan = o.plan;
  layout->bytes = o.plan + 4 * int64_t(info.plan_ints);
  layout->plan = info;
  return PKV_OK;
}

}  // extern "C"
