// PagedAttention decode for gfx950.
//
// For every sequence i and query head h: out = softmax(scale * q . K^T) . V
// over the sequence's logical tokens, with K/V rows read through the
// sequence's block table ("PagedAttention e continuous batching",
// 01 · Conceito, paragraph 3; "04 — Hacia PagedAttention", La idea de
// PagedAttention, step 5).  Paging changes where rows live, not the result
// or the FLOPs of dense attention ("Lo que deberías llevarte", item 2), so
// the kernel is bound by HBM bandwidth: one pass over the K/V bytes.
//
// Work decomposition.  A host plan cuts every sequence into partitions of P
// tokens (split-K); one workgroup takes one (partition, KV head, group of GW
// query heads sharing that KV head).  Its NW waves stride over the
// partition's blocks.  A (block, KV head) tile of K is 16 rows x R bytes,
// contiguous (R = head_dim * element size); lane l of a wave loads bytes
// [l*16, l*16+16) of each 1 KiB quarter, so every load instruction reads 1
// KiB contiguous.  With R = 256 (fp16/bf16 x 128, fp32 x 64) a row spans 16
// lanes, one DPP row: lanes of "row group" r = l/16 hold token rows r, r+4,
// r+8, r+12 of every block, each lane 8 (or 4) elements of each row.
//
// Per block and query head a lane forms the partial dot products of its
// chunk (v_dot2_f32_{f16,bf16} or fp32 FMA), sums them across the row's lanes
// with DPP rotations (all lanes of the row get the score), and updates an
// online softmax (running max m, running sum l, rescaled output o) that is
// private to its row group, so no cross-row exchange is needed inside the
// loop.  Scores are kept in base 2 (q . k * scale * log2 e) so that every
// exponential is one v_exp_f32.  The next block's K and V are loaded while
// the current one is processed: into a second register set, or, for fp16 /
// bf16 at head_dim 128 with one query head per workgroup, straight into a
// second LDS stage of the wave (buffer loads with the LDS bit).  K/V are
// read once per launch, so the loads carry the nontemporal hint: on MI355X
// that lifts the gather of the decode's 4 KiB tiles from 5.3-5.7 TB/s to
// 6.1-6.6 TB/s (pkv_gather_probe).  At the end the row groups and waves of the
// workgroup merge their (m, l, o) through LDS; a single-partition sequence
// writes o / l, otherwise (m, l, o) go to the workspace and the partitions
// are merged:  M = max m_p,
//   out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
// The merge runs in the same launch: each partial record is written with
// device-scope atomic stores, the workgroup waits for its stores, then takes
// a ticket from a per-(sequence, head) counter; the workgroup that takes the
// last ticket reads the records with device-scope loads, merges them and
// resets the counter to zero for the next launch.  pkv_paged_decode_reduce
// is the same merge as a kernel of its own.
//
// With k_new / v_new given, the sequence's newest token (position L-1) is
// taken from those arrays instead of the pool, and the workgroup of the first
// query-head group of its KV head stores it into its slot, so the decode and
// the append of that token are one launch.
//
// Rows past the sequence length in its last block are masked: their score
// is -inf and their V row is replaced by zeros, so stale or NaN contents of
// unused slots never reach the output.  Table entries outside the pool are
// treated as fully masked blocks (nothing is read through them).
#include <hip/hip_ext.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <mutex>
#include <string>
#include <type_traits>

#include "decode_launch.h"
#include "device_common.h"
#include "mfma_common.h"

namespace pkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct DecodeParams {
  const char* q;
  const char* k_new;           // [B][H_kv][D] newest token's K, or null
  const char* v_new;
  float* out;
  char* k_cache;
  char* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* work;         // [n_work][2] (sequence, partition)
  const int32_t* part_offset;  // [num_seqs] first partial index or -1
  const int32_t* priv_start;   // [num_seqs] first block of the sequence's own part, or null (0)
  const int32_t* n_shared;     // [num_seqs] records the shared launch wrote, or null (0)
  float* part;                 // [n_partials][H_q] records of rec_floats
  int32_t* counters;           // [num_seqs][H_q] completion tickets, or null
  int32_t rec_floats;          // record: o[D], m, l, padded to whole 128-byte lines
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;               // H_q / H_kv
  int32_t hgroups_per_kv;      // group / GW
  int32_t table_stride;
  int32_t num_blocks;
  int32_t partition_blocks;
  int32_t n_partials;
  float scale_log2;
};

// Split-K records are merged in batches: every load of a batch is issued
// before any is used, so their latencies overlap (a record-by-record loop
// waits for each load in turn, and a short item merging ten records spent
// most of its time there).
constexpr int kRecBatch = 8;

template <bool AGENT>
__device__ __forceinline__ float rec_load(const float* a) {
  if constexpr (AGENT) return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *a;
}

// Merge records rec0 + q * step, q < count, element dd, into the running
// state (M: base-2 maximum in scaled units, -inf for none; num, den scaled
// to it).  AGENT: records written in this launch (agent-scope loads);
// otherwise they come from an earlier launch and plain loads see them.
template <int D, bool AGENT>
__device__ __forceinline__ void merge_records(const float* rec0, int64_t step, int count, int dd, float& M,
                                              float& num, float& den) {
  for (int q0 = 0; q0 < count; q0 += kRecBatch) {
    float mq[kRecBatch], oq[kRecBatch], lq[kRecBatch];
#pragma unroll
    for (int i = 0; i < kRecBatch; ++i) {
      const bool ok = q0 + i < count;
      const float* rec = rec0 + int64_t(ok ? q0 + i : q0) * step;
      mq[i] = ok ? rec_load<AGENT>(rec + D) : -INFINITY;
      oq[i] = rec_load<AGENT>(rec + dd);
      lq[i] = rec_load<AGENT>(rec + D + 1);
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < kRecBatch; ++i) Mb = fmaxf(Mb, mq[i]);
    const float Mu = (Mb == -INFINITY) ? 0.f : Mb;
    const float a = __builtin_amdgcn_exp2f(M - Mu);
    num *= a;
    den *= a;
#pragma unroll
    for (int i = 0; i < kRecBatch; ++i) {
      const float w = (q0 + i < count) ? __builtin_amdgcn_exp2f(mq[i] - Mu) : 0.f;
      num = __builtin_fmaf(w, oq[i], num);
      den = __builtin_fmaf(w, lq[i], den);
    }
    M = Mb;
  }
}

// The end of a work item, shared by both decode kernels.  sm_m, sm_l
// ([NSUB][GW]) and sm_o ([NSUB][GW][D]) hold the workgroup's NSUB partial
// softmax states per query head (base-2 maxima in scaled units), written
// before a barrier.  They are merged.  A sequence owns n_sh records written
// by the shared launch (blocks it holds in common with others), then one
// per partition of its own blocks.
//  * one partition and no shared record: the item writes o / l;
//  * one partition and shared records (combine fused in): the item merges
//    its state with the shared records and writes the output;
//  * otherwise the partition's (o, m, l) becomes a record and the last
//    partition to finish combines all records of the (sequence, head group)
//    (without tickets, the two-launch variant, a separate kernel does).
template <int D, int GW, int NSUB, int NT>
__device__ __forceinline__ void finish_item(const DecodeParams& p, const float* sm_m, const float* sm_l,
                                            const float* sm_o, int seq, int part, int n_parts, int n_sh,
                                            int hg, int hgroups, int qh0) {
  const int n_rec = n_sh + n_parts;
  const bool single = (n_rec <= 1);
  const bool fold = (n_parts == 1 && n_sh > 0 && p.counters != nullptr);
  const int base = single ? -1 : p.part_offset[seq];
  if (!single && (base < 0 || base + n_rec > p.n_partials)) return;
  const int pidx = base + n_sh + part;
  const int64_t step = int64_t(p.num_q_heads) * p.rec_floats;
  for (int idx = threadIdx.x; idx < GW * D; idx += NT) {
    const int g = idx / D;
    const int dd = idx - g * D;
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) M = fmaxf(M, sm_m[s * GW + g]);
    const int qh = qh0 + g;
    const float M_use = (M == -INFINITY) ? 0.f : M;
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const float w = __builtin_amdgcn_exp2f(sm_m[s * GW + g] - M_use);
      num = __builtin_fmaf(w, sm_o[(s * GW + g) * D + dd], num);
      den = __builtin_fmaf(w, sm_l[s * GW + g], den);
    }
    if (fold) {
      // the shared records were written by the launch before this one
      const float* rec0 = p.part + (int64_t(base) * p.num_q_heads + qh) * p.rec_floats;
      merge_records<D, false>(rec0, step, n_sh, dd, M, num, den);
    }
    if (single || fold) {
      p.out[(int64_t(seq) * p.num_q_heads + qh) * D + dd] = num / den;
    } else {
      // partial record of (partition, query head): agent-scope stores, so
      // the combining workgroup on any XCD reads them without cache flushes
      float* rec = p.part + (int64_t(pidx) * p.num_q_heads + qh) * p.rec_floats;
      __hip_atomic_store(rec + dd, num, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (dd == 0) {
        __hip_atomic_store(rec + D, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(rec + D + 1, den, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (single || fold || p.counters == nullptr) return;

  // Split-K combine in the same launch.  Each workgroup of a (sequence, head
  // group) waits until its partial stores have completed, takes a ticket, and
  // the one taking the last ticket combines every record of the sequence
  // (shared ones included) and resets the ticket for the next launch.
  // Ordering.  Writer side: every thread's record stores are agent-scope
  // atomic stores, waited for (s_waitcnt) before the workgroup barrier, and
  // the barrier orders them before thread 0's ticket add; the records are
  // therefore performed at agent scope before the ticket can count them.
  // No release fence is added there: at agent scope it writes back the
  // whole L2 of the compute unit's XCD, in every workgroup of every split
  // sequence.  Reader side: the workgroup that draws the last ticket takes
  // an agent-scope acquire fence before the barrier that releases its
  // threads to read the records (agent-scope atomic loads), so no load of a
  // record can be satisfied before the ticket was observed.
  __shared__ int sm_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int32_t* ticket = p.counters + int64_t(seq) * hgroups + hg;
  if (threadIdx.x == 0) {
    const bool last =
        __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_parts - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    sm_last = last;
  }
  __syncthreads();
  if (!sm_last) return;
  for (int idx = threadIdx.x; idx < GW * D; idx += NT) {
    const int g = idx / D;
    const int dd = idx - g * D;
    const int qh = qh0 + g;
    const float* rec0 = p.part + (int64_t(base) * p.num_q_heads + qh) * p.rec_floats;
    float M = -INFINITY, num = 0.f, den = 0.f;
    merge_records<D, true>(rec0, step, n_rec, dd, M, num, den);
    p.out[(int64_t(seq) * p.num_q_heads + qh) * D + dd] = num / den;
  }
  if (threadIdx.x == 0) __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Occupancy hint (waves per SIMD) where the compiler fits the kernel in
// the matching register budget without spilling (checked per instance):
// 4 (128 registers) for bf16 x 128 with one head per workgroup, 3 (168) for
// fp16 x 128 with one head and bf16 x 128 with two; else none.
template <int DT, int D, int GW>
constexpr int decode_waves_hint() {
  if (D != 128) return 1;
  if (DT == PKV_BF16) return GW == 1 ? 4 : GW == 2 ? 3 : 1;
  if (DT == PKV_F16) return GW == 1 ? 3 : 1;
  return 1;
}

// Cache policy of the K/V tile loads.  Tiles that one launch reads once go
// nontemporal (kCacheStream, as load_stream): that raises the rate of the
// scattered tile reads.  When sequences of the batch share blocks (forked
// prefixes), many workgroups read the same tiles at about the same time and
// ordinary loads (kCacheReuse) let L2 serve the repeats; the nontemporal
// policy evicts those lines first, and every repeat goes back to the fabric.
constexpr int kCacheStream = kCachePolicyNT;
constexpr int kCacheReuse = 0;

template <int CP>
__device__ __forceinline__ u32x4 load_tile(__amdgpu_buffer_rsrc_t r, int offset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, CP));
}

// LDS: stage K/V tiles through LDS instead of registers (see the main loop
// and lds_staging).
template <int DT, int D, int GW, int NW, int CP = kCacheStream, bool LDS = false>
__global__ __launch_bounds__(kWave* NW, (LDS ? 2 : decode_waves_hint<DT, D, GW>())) void paged_decode_kernel(
    const DecodeParams p) {
  constexpr int E = ElemBytes<DT>::value;
  constexpr int R = D * E;         // bytes per token row of one head
  constexpr int LPR = R / 16;      // lanes per token row
  constexpr int RPI = kWave / LPR; // token rows per load instruction
  constexpr int NI = kBlockTokens / RPI;  // load instructions per tile
  constexpr int EPL = 16 / E;      // elements per lane per row
  constexpr int TILE = kBlockTokens * R;
  static_assert(LPR >= 8 && LPR <= 64 && NI >= 1, "unsupported head_dim / dtype");

  __shared__ float sm_m[NW * RPI * GW];
  __shared__ float sm_l[NW * RPI * GW];
  __shared__ float sm_o[NW * RPI * GW * D];
  // LDS staging ring: two stages (K and V of one block each) per wave, as
  // two distinct arrays, so that the wait before reading one stage leaves
  // the loads into the other in flight
  constexpr int SW = LDS ? NW : 1;
  constexpr int SB = LDS ? 2 * TILE : 16;
  __shared__ __attribute__((aligned(16))) char st_a[SW][SB];
  __shared__ __attribute__((aligned(16))) char st_b[SW][SB];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int hgroups = p.num_kv_heads * p.hgroups_per_kv;
  const int wi = blockIdx.x / hgroups;
  const int hg = blockIdx.x - wi * hgroups;
  const int seq = p.work[2 * wi];
  const int part = p.work[2 * wi + 1];
  const int kvh = hg / p.hgroups_per_kv;
  const int qh0 = kvh * p.group + (hg - kvh * p.hgroups_per_kv) * GW;
  const int L = p.context_lens[seq];
  const int nblk = min((L + kBlockTokens - 1) / kBlockTokens, p.table_stride);
  const int ps = p.priv_start ? p.priv_start[seq] : 0;  // blocks before it: shared launch
  const int n_sh = p.n_shared ? p.n_shared[seq] : 0;
  const int n_parts = (nblk - ps + p.partition_blocks - 1) / p.partition_blocks;
  const int b0 = ps + part * p.partition_blocks;
  const int b1 = min(b0 + p.partition_blocks, nblk);

  const int rg = lane / LPR;  // row group
  const int c = lane - rg * LPR;
  const bool writes_new = (hg - kvh * p.hgroups_per_kv) == 0;

  u32x4 qv[GW];
#pragma unroll
  for (int g = 0; g < GW; ++g)
    qv[g] = *reinterpret_cast<const u32x4*>(
        p.q + (int64_t(seq) * p.num_q_heads + qh0 + g) * R + c * 16);

  float m[GW], l[GW], o[GW][EPL];
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[g][e] = 0.f;
  }

  const int32_t* trow = p.block_tables + int64_t(seq) * p.table_stride;
  const int64_t blk_stride = int64_t(p.num_kv_heads) * TILE;

  // Issue the K/V loads of block j of the current chunk (see below).  The
  // loads are always issued, so every path through the loop has the same
  // loads in flight and each wait covers exactly the buffer about to be used;
  // past the chunk's end, or for a table entry outside the pool, the buffer
  // resource has no records and the loads return zeros without touching
  // memory.  Returns the block id.
  int cb = 0, ce = 0, tbl = -1;
  auto issue = [&](int j, u32x4* kk, u32x4* vv) __attribute__((always_inline)) -> int {
    const int blk = __builtin_amdgcn_readlane(tbl, min(j - cb, kWave - 1));
    const bool ok = j < ce && unsigned(blk) < unsigned(p.num_blocks);
    const int64_t tile = int64_t(ok ? blk : 0) * blk_stride + int64_t(kvh) * TILE;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k_cache + tile, ok ? TILE : 0);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v_cache + tile, ok ? TILE : 0);
#pragma unroll
    for (int i = 0; i < NI; ++i) kk[i] = load_tile<CP>(rk, lane * 16 + i * 1024);
#pragma unroll
    for (int i = 0; i < NI; ++i) vv[i] = load_tile<CP>(rv, lane * 16 + i * 1024);
    return j < ce ? blk : -1;
  };

  // Online-softmax update with one block; `valid` = rows of the block that
  // hold tokens (16 except in the last block).
  auto process = [&](const u32x4* kk, const u32x4* vv, int valid, bool masked) __attribute__((always_inline)) {
    float ps[GW][NI];
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      float s[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float part_dot = dot16<DT>(qv[g], kk[i], 0.f);
        s[i] = row_sum<LPR>(part_dot) * p.scale_log2;
      }
      if (masked) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
          if (i * RPI + rg >= valid) s[i] = -INFINITY;
      }
      float mx = s[0];
#pragma unroll
      for (int i = 1; i < NI; ++i) mx = fmaxf(mx, s[i]);
      const float m_new = fmaxf(m[g], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m[g] - m_use);
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        ps[g][i] = __builtin_amdgcn_exp2f(s[i] - m_use);
        sum += ps[g][i];
      }
      l[g] = l[g] * alpha + sum;
      m[g] = m_new;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[g][e] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float vf[EPL];
      to_f32<DT>(vv[i], vf);
      if (masked && i * RPI + rg >= valid) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int g = 0; g < GW; ++g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[g][e] = __builtin_fmaf(ps[g][i], vf[e], o[g][e]);
    }
  };

  // The sequence's newest token, held in registers (nk, nv: this lane's
  // chunk of its K and V rows), as one more online-softmax update.  Every
  // row group computes the score; only row group 0 counts the token.
  auto process_one = [&](const u32x4& nk, const u32x4& nv) __attribute__((always_inline)) {
    float vf[EPL];
    to_f32<DT>(nv, vf);
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      float sc = row_sum<LPR>(dot16<DT>(qv[g], nk, 0.f)) * p.scale_log2;
      if (rg != 0) sc = -INFINITY;
      const float m_new = fmaxf(m[g], sc);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m[g] - m_use);
      const float pn = __builtin_amdgcn_exp2f(sc - m_use);
      l[g] = l[g] * alpha + pn;
      m[g] = m_new;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[g][e] = __builtin_fmaf(pn, vf[e], o[g][e] * alpha);
    }
  };

  // One block.  The last block of the sequence is masked past its length.
  // With k_new given, the newest token (position L-1, row r_new of the last
  // block) comes from k_new/v_new instead of the pool: the block is processed
  // without that row, the row as process_one, and the first head group of
  // the KV head stores it into the pool.
  auto consume = [&](const u32x4* kk, const u32x4* vv, int j, int blk) __attribute__((always_inline)) {
    const bool in_pool = unsigned(blk) < unsigned(p.num_blocks);
    if (in_pool && j != nblk - 1) {
      process(kk, vv, kBlockTokens, false);
      return;
    }
    const int r_new = L - 1 - j * kBlockTokens;
    if (p.k_new != nullptr && in_pool && r_new >= 0 && r_new < kBlockTokens) {
      const int64_t src = (int64_t(seq) * p.num_kv_heads + kvh) * R + c * 16;
      const u32x4 nk = *reinterpret_cast<const u32x4*>(p.k_new + src);
      const u32x4 nv = *reinterpret_cast<const u32x4*>(p.v_new + src);
      if (writes_new && rg == r_new % RPI) {
        const int64_t dst = int64_t(blk) * blk_stride + int64_t(kvh) * TILE + int64_t(r_new) * R + c * 16;
        *reinterpret_cast<u32x4*>(p.k_cache + dst) = nk;
        *reinterpret_cast<u32x4*>(p.v_cache + dst) = nv;
      }
      process(kk, vv, r_new, true);
      process_one(nk, nv);
      return;
    }
    const int valid = in_pool ? min(kBlockTokens, L - j * kBlockTokens) : 0;
    process(kk, vv, valid, true);
  };

  // Wave `wave` takes blocks b0 + wave, b0 + wave + NW, ...  The partition's
  // table entries come in chunks of 64, one entry per lane, loaded once per
  // chunk; inside a chunk a block id is a v_readlane, so the only memory
  // operations in the inner loop are the K/V loads.  Two register buffers
  // alternate: the next block loads while the current one computes.
  u32x4 ka[NI], va[NI], kb[NI], vb[NI];
  if constexpr (!LDS) {
    for (cb = b0; cb < b1; cb += kWave) {
      ce = min(cb + kWave, b1);
      tbl = (cb + lane < ce) ? trow[cb + lane] : -1;
      int j = cb + wave;
      if (j >= ce) break;  // uniform: no block of this chunk (nor later ones) for this wave
      int blk_a = issue(j, ka, va), blk_b;
      while (true) {
        blk_b = issue(j + NW, kb, vb);
        consume(ka, va, j, blk_a);
        j += NW;
        if (j >= ce) break;
        blk_a = issue(j + NW, ka, va);
        consume(kb, vb, j, blk_b);
        j += NW;
        if (j >= ce) break;
      }
    }
  } else {
    // The same walk with the tiles loaded straight into the wave's LDS ring
    // (buffer loads with the LDS bit: lane l's 16 bytes of load i land at
    // byte 1024 i + 16 l of the stage, the tile's own layout), then read
    // back into the same register layout and processed as above.  No
    // registers hold loads in flight, but a stage costs 8 KiB of LDS per
    // wave: 72 KiB per workgroup of four waves, two workgroups per CU.
    auto stage_in = [&](auto stage, int j) __attribute__((always_inline)) -> int {
      const int blk = __builtin_amdgcn_readlane(tbl, min(j - cb, kWave - 1));
      const bool ok = j < ce && unsigned(blk) < unsigned(p.num_blocks);
      const int64_t tile = int64_t(ok ? blk : 0) * blk_stride + int64_t(kvh) * TILE;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k_cache + tile, ok ? TILE : 0);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v_cache + tile, ok ? TILE : 0);
      char* base = decltype(stage)::value == 0 ? &st_a[wave][0] : &st_b[wave][0];
#pragma unroll
      for (int i = 0; i < NI; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(base + i * 1024),
                                                 16, lane * 16 + i * 1024, 0, 0, CP);
#pragma unroll
      for (int i = 0; i < NI; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (__attribute__((address_space(3))) void*)(base + TILE + i * 1024), 16, lane * 16 + i * 1024, 0, 0, CP);
      return j < ce ? blk : -1;
    };
    auto stage_out = [&](auto stage, u32x4* kk, u32x4* vv) __attribute__((always_inline)) {
      const char* base = decltype(stage)::value == 0 ? &st_a[wave][0] : &st_b[wave][0];
#pragma unroll
      for (int i = 0; i < NI; ++i) kk[i] = *reinterpret_cast<const u32x4*>(base + i * 1024 + lane * 16);
#pragma unroll
      for (int i = 0; i < NI; ++i) vv[i] = *reinterpret_cast<const u32x4*>(base + TILE + i * 1024 + lane * 16);
    };
    using StA = std::integral_constant<int, 0>;
    using StB = std::integral_constant<int, 1>;
    for (cb = b0; cb < b1; cb += kWave) {
      ce = min(cb + kWave, b1);
      tbl = (cb + lane < ce) ? trow[cb + lane] : -1;
      int j = cb + wave;
      if (j >= ce) break;
      int blk_a = stage_in(StA{}, j), blk_b;
      while (true) {
        blk_b = stage_in(StB{}, j + NW);
        stage_out(StA{}, ka, va);
        consume(ka, va, j, blk_a);
        j += NW;
        if (j >= ce) break;
        blk_a = stage_in(StA{}, j + NW);
        stage_out(StB{}, kb, vb);
        consume(kb, vb, j, blk_b);
        j += NW;
        if (j >= ce) break;
      }
    }
  }

  // merge the NW * RPI partial softmax states of this workgroup
  const int sub = wave * RPI + rg;
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    if (c == 0) {
      sm_m[sub * GW + g] = m[g];
      sm_l[sub * GW + g] = l[g];
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) sm_o[(sub * GW + g) * D + c * EPL + e] = o[g][e];
  }
  __syncthreads();

  finish_item<D, GW, NW * RPI, kWave * NW>(p, sm_m, sm_l, sm_o, seq, part, n_parts, n_sh, hg, hgroups, qh0);
}

// ---------------------------------------------------------------------------
// Grouped-query decode on the matrix cores (fp16 / bf16, head_dim 128).
//
// With GQA the GW query heads of a KV head share every K/V tile, so per
// block S^T = K Q^T is a 16-token x GW-head product and O^T += V^T P^T a
// 128-dim x GW-head one: small dense contractions that the VALU path spends
// about 400 instructions per tile on (dot products, row sums, per-head
// softmax, per-head V products).  Here they run as MFMA, with GW heads in
// the 16 columns (column n serves head n mod GW; the copies cost nothing
// on the matrix cores, and every lane then holds a real head).
//
// Lane (g, n) = lane (16 g + n).  Per block and wave:
//  * K tile: four loads of 1 KiB (tokens 4 i .. 4 i + 3) straight into the
//    wave's LDS stage (buffer loads with the LDS bit), each token row's
//    16-byte chunks permuted (chunk c of token t at position c ^ t); the wave
//    reads back, for k-step kc, dims 32 kc + 8 g .. + 7 of token n: the A
//    operand of v_mfma_f32_16x16x32 (row n, k-slice 8 g).  (Loading that
//    layout straight from HBM into registers takes 16 rows x 64 bytes per
//    load, measured 3.6% slower than staging.)  Q^T is the B operand
//    (column n, the same dims), loaded once.
//  * The accumulator leaves lane (g, n) with the scores of tokens
//    4 g .. 4 g + 3 for column n: the B-operand layout of the 16x16x16
//    product that follows, so the weights never move between lanes.  The
//    online softmax keeps one running maximum per column and a per-lane
//    partial sum; the maximum lags the column's by up to kDecodeSlack, and
//    the four lanes of a column exchange their maxima (gfx950's lane swaps)
//    only in a block where one lane's scores pass it by more than that.
//  * V tile: load j (j = 0..3) gives lane (g, n) dims 8 n .. 8 n + 7 of
//    token 4 g + j, four full 256-byte rows per load.  The lane then holds
//    its four tokens at eight dims; pairing halves gives, for each dim
//    8 n + t (t = 0..7), the A operand of O^T += V^T P^T (row n, tokens
//    4 g .. 4 g + 3), so d-tile t of O^T covers dims 8 r + t for rows r and
//    lane (g, n) ends with dims 32 g .. 32 g + 31 of its column: no LDS
//    transpose.
//  * Weights: fp16 inputs round them to fp16; bf16 inputs split them into a
//    bf16 head and a bf16 remainder (two products), since bf16 weights
//    alone put short contexts above the 2e-3 tolerance.  The normaliser
//    sums the weights the products use: the fp16-rounded ones, or the fp32
//    ones for bf16 (head + remainder match them to ~16 bits).
//  * Masking: the tile's buffer resources cover only the rows that hold
//    tokens (zeros beyond, so V rows past the length contribute 0 even if
//    the pool holds NaN there) and scores of rows past the length are -inf.
//  * With k_new / v_new, the newest token's row is taken from those arrays
//    into the registers of the tile (the pool slot may still be being
//    written by this launch), and the first head group stores it.
// The partition's states then merge and combine as in the VALU kernel.
// Slack of the matrix-core decode's running maxima, in base-2 units: a
// column's maximum is raised (and its accumulators rescaled) only when a score
// exceeds it by more than this, so after the first keys the rescale almost
// never runs; weights stay <= 2^8, exact enough as fp16 or as a bf16 head
// plus remainder.
constexpr float kDecodeSlack = 8.f;

// A 16-byte tile load (cache policy CP, as load_tile) whose wave-uniform part
// of the offset sits in a scalar register, so that one vector offset serves
// all loads of a tile.
template <int CP>
__device__ __forceinline__ u32x4 load_tile_s(__amdgpu_buffer_rsrc_t r, int voffset, int soffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, soffset, CP));
}

template <int DT, int GW, int NW, int CP = kCacheStream>
__global__ __launch_bounds__(kWave* NW, 3) void paged_decode_mfma_kernel(const DecodeParams p) {
  constexpr int D = 128;
  constexpr int R = D * 2;                // bytes per token row of one head
  constexpr int TILE = kBlockTokens * R;  // one (block, KV head) tile
  static_assert(GW >= 2 && GW <= 16 && (GW & (GW - 1)) == 0, "2 to 16 heads per workgroup");
  static_assert(DT == PKV_F16 || DT == PKV_BF16, "16-bit inputs");

  __shared__ float sm_m[NW * GW];
  __shared__ float sm_l[NW * GW];
  __shared__ __attribute__((aligned(16))) float sm_o[NW * GW * D];
  // K tiles go straight from HBM into LDS (buffer loads with the LDS bit),
  // into a ring of two stages per wave held in two distinct arrays, so that
  // the compiler's wait before reading one stage leaves the other's loads in
  // flight.  A load writes lane l's 16 bytes at byte 16 l of its 1 KiB; the
  // lane loads the chunk that belongs there: token t's 16-byte chunk c sits
  // at position c ^ (t mod 16) of row t, so that the operand reads below
  // (16 lanes: 16 tokens, one chunk each) hit distinct banks.
  __shared__ __attribute__((aligned(16))) char sk_a[NW][TILE];
  __shared__ __attribute__((aligned(16))) char sk_b[NW][TILE];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane >> 4;
  const int n = lane & 15;
  const int hgroups = p.num_kv_heads * p.hgroups_per_kv;
  const int wi = blockIdx.x / hgroups;
  const int hg = blockIdx.x - wi * hgroups;
  const int seq = p.work[2 * wi];
  const int part = p.work[2 * wi + 1];
  const int kvh = hg / p.hgroups_per_kv;
  const int qh0 = kvh * p.group + (hg - kvh * p.hgroups_per_kv) * GW;
  const int L = p.context_lens[seq];
  const int nblk = min((L + kBlockTokens - 1) / kBlockTokens, p.table_stride);
  const int ps = p.priv_start ? p.priv_start[seq] : 0;  // blocks before it: shared launch
  const int n_sh = p.n_shared ? p.n_shared[seq] : 0;
  const int n_parts = (nblk - ps + p.partition_blocks - 1) / p.partition_blocks;
  const int b0 = ps + part * p.partition_blocks;
  const int b1 = min(b0 + p.partition_blocks, nblk);
  const bool writes_new = (hg - kvh * p.hgroups_per_kv) == 0;
  const float c2 = p.scale_log2;

  // Q^T (B operand): column n = head qh0 + n mod GW, dims 32 kc + 8 g .. + 7
  u32x4 qb[4];
  {
    const char* qrow = p.q + (int64_t(seq) * p.num_q_heads + qh0 + (n & (GW - 1))) * R;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) qb[kc] = *reinterpret_cast<const u32x4*>(qrow + 64 * kc + 16 * g);
  }

  float m = kNegBig, lsum = 0.f;
  f4 o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = f4{0.f, 0.f, 0.f, 0.f};

  const int32_t* trow = p.block_tables + int64_t(seq) * p.table_stride;
  const int64_t blk_stride = int64_t(p.num_kv_heads) * TILE;

  // Issue the K/V loads of block j of the current chunk into kk / vv.  The
  // loads are always issued (same loads on every path, exact vmcnt waits);
  // the resources cover the rows that hold tokens, none past the chunk's
  // end or for a table entry outside the pool.  Returns the block id.
  int cb = 0, ce = 0, tbl = -1;
  int koff[4];  // load i: token 4 i + g, the chunk stored at position n
#pragma unroll
  for (int i = 0; i < 4; ++i) koff[i] = (4 * i + g) * R + 16 * (n ^ (4 * i + g));
  const int voff = 4 * g * R + 16 * n;  // + t R
  auto kstage = [&](auto sc) __attribute__((always_inline)) -> char* {
    return decltype(sc)::value == 0 ? &sk_a[wave][0] : &sk_b[wave][0];
  };
  auto issue = [&](auto sc, int j, u32x4* vv) __attribute__((always_inline)) -> int {
    const int blk = __builtin_amdgcn_readlane(tbl, min(j - cb, kWave - 1));
    const bool ok = j < ce && unsigned(blk) < unsigned(p.num_blocks);
    const int rows = ok ? min(kBlockTokens, L - j * kBlockTokens) : 0;
    const int64_t tile = int64_t(ok ? blk : 0) * blk_stride + int64_t(kvh) * TILE;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k_cache + tile, rows * R);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v_cache + tile, rows * R);
    char* dst = kstage(sc);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16,
                                               koff[i], 0, 0, CP);
#pragma unroll
    for (int t = 0; t < 4; ++t) vv[t] = load_tile_s<CP>(rv, voff, t * R);
    return j < ce ? blk : -1;
  };

  // One block: `valid` rows hold tokens (16 except in the last block).
  // K comes from the wave's LDS stage as the A operand (row n, dims
  // 32 kc + 8 g); with `knew`, lanes of row r_new take it from kn instead
  // (the newest token, not read from the pool).
  auto process = [&](const char* klds, const u32x4* vv, int valid, bool knew, int r_new,
                     const u32x4* kn) __attribute__((always_inline)) {
    f4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      u32x4 a = *reinterpret_cast<const u32x4*>(klds + n * R + 16 * ((4 * kc + g) ^ n));
      if (knew) a = n == r_new ? kn[kc] : a;
      sacc = mfma_k32<DT>(a, qb[kc], sacc);
    }
    float s[4] = {sacc[0], sacc[1], sacc[2], sacc[3]};
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r >= valid) s[r] = -INFINITY;
    // the running maximum moves only when a score exceeds it by more than
    // kDecodeSlack (weights stay <= 2^kDecodeSlack in between); the lane's
    // own scores decide whether any of the column's can, so the column's
    // maximum over its four lanes, the factor and the accumulators' rescale
    // are formed only in such a block
    const float mxl = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    float alpha = 1.f;
    if (__builtin_amdgcn_ballot_w64(mxl * c2 > m + kDecodeSlack)) {
      const float mxs = max_over_lane_groups(mxl) * c2;
      const float mn = mxs > m + kDecodeSlack ? mxs : m;
      alpha = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
#pragma unroll
      for (int t = 0; t < 8; ++t) o[t] *= alpha;
    }
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c2, -m));
    const f2 x01 = {x[0], x[1]}, x23 = {x[2], x[3]};
    u32x2 pb, pl;
    if constexpr (DT == PKV_F16) {
      // the normaliser sums the weights as rounded (one dot product per pair)
      const h2 h01 = __builtin_convertvector(x01, h2), h23 = __builtin_convertvector(x23, h2);
      pb = u32x2{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)};
      lsum = lsum * alpha + __builtin_amdgcn_fdot2(h23, h2{1.f16, 1.f16},
                                                   __builtin_amdgcn_fdot2(h01, h2{1.f16, 1.f16}, 0.f, false), false);
    } else {
      lsum = lsum * alpha + ((x[0] + x[1]) + (x[2] + x[3]));
      const b2 h01 = __builtin_convertvector(x01, b2), h23 = __builtin_convertvector(x23, b2);
      pb = u32x2{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)};
      pl = u32x2{__builtin_bit_cast(uint32_t, __builtin_convertvector(x01 - __builtin_convertvector(h01, f2), b2)),
                 __builtin_bit_cast(uint32_t, __builtin_convertvector(x23 - __builtin_convertvector(h23, f2), b2))};
    }
    // vv[j] word w holds dims 8 n + 2 w (low half) and 8 n + 2 w + 1 (high
    // half) of token 4 g + j
    const uint32_t v0[4] = {vv[0].x, vv[0].y, vv[0].z, vv[0].w};
    const uint32_t v1[4] = {vv[1].x, vv[1].y, vv[1].z, vv[1].w};
    const uint32_t v2[4] = {vv[2].x, vv[2].y, vv[2].z, vv[2].w};
    const uint32_t v3[4] = {vv[3].x, vv[3].y, vv[3].z, vv[3].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u32x2 lo = {(v0[w] & 0xFFFFu) | (v1[w] << 16), (v2[w] & 0xFFFFu) | (v3[w] << 16)};
      const u32x2 hi = {(v0[w] >> 16) | (v1[w] & 0xFFFF0000u), (v2[w] >> 16) | (v3[w] & 0xFFFF0000u)};
      o[2 * w] = mfma_k16<DT>(lo, pb, o[2 * w]);
      o[2 * w + 1] = mfma_k16<DT>(hi, pb, o[2 * w + 1]);
      if constexpr (DT == PKV_BF16) {
        o[2 * w] = mfma_k16<DT>(lo, pl, o[2 * w]);
        o[2 * w + 1] = mfma_k16<DT>(hi, pl, o[2 * w + 1]);
      }
    }
  };

  // One block.  Rows past the sequence length (in its last block) or in a
  // table entry outside the pool are masked; every block takes the same
  // masked step (a few compares), which keeps one copy of the step per
  // stage.  With k_new given, the newest row (position L - 1) replaces row
  // r_new of the tile: K as the A operand of the lanes of row r_new (dims
  // 32 kc + 8 g, loaded here), V in lane group r_new / 4 of load r_new mod
  // 4; the first head group stores it.
  auto consume = [&](auto sc, u32x4* vv, int j, int blk) __attribute__((always_inline)) {
    const bool in_pool = unsigned(blk) < unsigned(p.num_blocks);
    const int valid = in_pool ? min(kBlockTokens, L - j * kBlockTokens) : 0;
    const int r_new = L - 1 - j * kBlockTokens;
    if (p.k_new != nullptr && in_pool && r_new < kBlockTokens) {
      // (a path of its own: the other blocks' operand reads then share no
      // registers with these loads, and never wait for them)
      const int64_t src = (int64_t(seq) * p.num_kv_heads + kvh) * R;
      const u32x4 nv = *reinterpret_cast<const u32x4*>(p.v_new + src + 16 * n);
      const u32x4 nk = *reinterpret_cast<const u32x4*>(p.k_new + src + 16 * n);
      u32x4 kn[4];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) kn[kc] = *reinterpret_cast<const u32x4*>(p.k_new + src + 16 * (4 * kc + g));
#pragma unroll
      for (int t = 0; t < 4; ++t) vv[t] = (g == (r_new >> 2) && t == (r_new & 3)) ? nv : vv[t];
      if (writes_new && g == 0) {
        const int64_t dst = int64_t(blk) * blk_stride + int64_t(kvh) * TILE + int64_t(r_new) * R + 16 * n;
        *reinterpret_cast<u32x4*>(p.k_cache + dst) = nk;
        *reinterpret_cast<u32x4*>(p.v_cache + dst) = nv;
      }
      process(kstage(sc), vv, valid, true, r_new, kn);
    } else {
      process(kstage(sc), vv, valid, false, -1, nullptr);
    }
  };

  // Wave `wave` takes blocks b0 + wave, b0 + wave + NW, ... (table entries in
  // chunks of 64, one per lane; two register buffers alternate, as in the
  // VALU kernel).
  using StA = std::integral_constant<int, 0>;
  using StB = std::integral_constant<int, 1>;
  u32x4 va[4], vb[4];
  for (cb = b0; cb < b1; cb += kWave) {
    ce = min(cb + kWave, b1);
    tbl = (cb + lane < ce) ? trow[cb + lane] : -1;
    int j = cb + wave;
    if (j >= ce) break;
    int blk_a = issue(StA{}, j, va), blk_b;
    while (true) {
      blk_b = issue(StB{}, j + NW, vb);
      consume(StA{}, va, j, blk_a);
      j += NW;
      if (j >= ce) break;
      blk_a = issue(StA{}, j + NW, va);
      consume(StB{}, vb, j, blk_b);
      j += NW;
      if (j >= ce) break;
    }
  }

  // this wave's state per column: the sum over the four lane groups, dims
  // 32 g + 8 r + t in o[t][r]
  float lt = lsum + __shfl_xor(lsum, 16);
  lt += __shfl_xor(lt, 32);
  if (n < GW) {
    if (g == 0) {
      sm_m[wave * GW + n] = m;
      sm_l[wave * GW + n] = lt;
    }
    float* orow = sm_o + (wave * GW + n) * D + 32 * g;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *reinterpret_cast<f4*>(orow + 8 * r) = f4{o[0][r], o[1][r], o[2][r], o[3][r]};
      *reinterpret_cast<f4*>(orow + 8 * r + 4) = f4{o[4][r], o[5][r], o[6][r], o[7][r]};
    }
  }
  __syncthreads();

  finish_item<D, GW, NW, kWave * NW>(p, sm_m, sm_l, sm_o, seq, part, n_parts, n_sh, hg, hgroups, qh0);
}

// ---------------------------------------------------------------------------
// Shared-block decode (fp16 / bf16, head_dim 128): blocks held in common by
// several sequences of the batch, read once for all of them.
//
// Forked sequences point at the same read-only blocks ("PagedAttention e
// continuous batching", 01 · Conceito, paragraph 6).  The host plan groups
// such sequences into nodes (a run of blocks every member holds at the same
// table positions) and cuts each node into chunks of blocks and column sets
// of members.  One workgroup takes one (chunk, column set, KV head): its
// columns are the (member, query head) pairs of the set that read this KV
// head, up to 128, so S^T = K Q^T (16 tokens x 16 columns per product) and
// O^T += V^T P^T are dense products for the matrix cores even where every
// sequence has a single query head (MHA): the chunk's keys serve all those
// queries at once, as a chunked prefill's keys serve a tile of query rows.
//
// Keys stream in stages of 32 tokens (two blocks), double-buffered in LDS:
// all 256 threads load the next stage into registers (every load
// instruction 1 KiB contiguous; each wave's rows lie in one block) while
// the current one is computed, then store K rows as they are and V
// transposed (dim-major, 4-token column blocks XOR-swizzled by bits 5-6 of
// the dim: the staging stores hit distinct banks and the operand reads stay
// 8-byte contiguous).  Wave w holds column groups 2w and 2w + 1 (16 columns
// each): every K operand read from LDS feeds both groups' S^T products, the
// accumulator (tokens 4g .. 4g + 3 of column n in lane 16 g + n, for each of
// the stage's two blocks) is the B operand of the 16x16x32 product
// O^T += V^T P^T over the stage's 32 tokens, and every V^T operand feeds
// both groups' products.  Online softmax per column in base 2 with the
// scale folded into the exponent; a column's running maximum moves only
// when a score passes it by more than 2^8 in weight, so after the first
// keys the accumulators are almost never rescaled.  Softmax weights enter
// the products as fp16 (fp16 inputs) or a bf16 head plus a bf16 remainder
// (bf16 inputs); the normaliser sums the weights the products use (the
// fp16-rounded ones; the fp32 ones for bf16).
// Every block in a node is full in every member (a sequence's last block is
// never shared); a stage's second block past the chunk, or a table entry
// outside the pool, reads nothing and its keys are masked.
// Each column's (o, m, l) becomes the split-K record of its (member, query
// head) for this chunk; the decode launch that follows merges them with
// the member's own blocks.
constexpr int kNodeInts = 9;  // rep, j0, j1, first member, members, first record, first item, column sets, chunk

struct SharedParams {
  const char* q;
  const char* k_cache;
  const char* v_cache;
  const int32_t* block_tables;
  const int32_t* part_offset;  // [num_seqs] first record of each sequence
  const int32_t* order;        // [num_seqs] batch indices, node members contiguous
  const int32_t* nodes;        // [n_nodes][kNodeInts]
  float* part;
  int32_t rec_floats;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t table_stride;
  int32_t num_blocks;
  int32_t n_nodes;
  int32_t per_set;  // members per column set: kSharedCols / group
  int32_t n_partials;
  float scale_log2;
};

constexpr int kSharedRG = 2;                       // 16-column groups per wave
constexpr int kSharedCols = 4 * kSharedRG * 16;    // columns per workgroup
constexpr int kSharedStage = 32;                   // tokens per LDS stage (two blocks)
constexpr float kSharedSlack = 8.f;                // log2 of the weight a running maximum may lag

// WPS: waves per SIMD the register budget is fitted to (2 or 3).
template <int DT, int CP, int WPS>
__global__ __launch_bounds__(256, WPS) void paged_decode_shared_kernel(const SharedParams p) {
  constexpr int D = 128;
  constexpr int RG = kSharedRG;
  constexpr int CH = D / 8;                 // 16-byte chunks per token row
  constexpr int ROWB = D * 2;
  constexpr int TILE = kBlockTokens * ROWB;
  constexpr int KROW = D + 8;               // K row stride in LDS (16-bit elements)
  constexpr int VROW = kSharedStage + 4;    // V^T row stride in LDS
  constexpr int KL = kSharedStage * CH / 256;  // K chunks each thread stages
  constexpr int NDT = D / 16;
  static_assert(KL == 2 && CH * (kSharedStage / 2) == 256, "staging split");
  // V^T column of stage token tok in LDS row r (a dim); see the comment above
  auto vt_col = [](int r, int tok) __attribute__((always_inline)) {
    return (((tok >> 2) ^ (2 * ((r >> 5) & 3))) << 2) | (tok & 3);
  };
  __shared__ __attribute__((aligned(16))) uint16_t lk[2][kSharedStage * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t lv[2][D * VROW];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane >> 4;
  const int n = lane & 15;
  const int item = blockIdx.x / p.num_kv_heads;
  const int kvh = blockIdx.x - item * p.num_kv_heads;

  // the node holding this item: the last one whose first item is <= item
  int lo = 0, hi = p.n_nodes - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.nodes[kNodeInts * mid + 6] <= item) lo = mid;
    else hi = mid - 1;
  }
  const int32_t* nd = p.nodes + kNodeInts * lo;
  const int rep = nd[0], j0 = nd[1], j1 = nd[2], first = nd[3], members = nd[4], k_base = nd[5];
  const int colsets = nd[7];
  const int local = item - nd[6];
  const int chunk = local / colsets;
  const int cset = local - chunk * colsets;
  const int b0 = j0 + chunk * nd[8];
  const int b1 = min(j1, b0 + nd[8]);
  const int nst = (b1 - b0 + 1) >> 1;  // stages; the last may hold one block
  const int m0 = cset * p.per_set;
  const int cols = min(p.per_set, members - m0) * p.group;
  const float c2 = p.scale_log2;

  // this lane's columns: group j is columns (RG wave + j) * 16 + n of the
  // set, a (member, query head) pair each; columns past the set repeat its
  // first one and write nothing
  auto column = [&](int j, int& mem, int& qh) __attribute__((always_inline)) -> bool {
    const int c = (RG * wave + j) * 16 + n;
    const int cc = c < cols ? c : 0;
    mem = p.order[first + m0 + cc / p.group];
    qh = kvh * p.group + (cc - (cc / p.group) * p.group);
    return c < cols;
  };
  u32x4 qb[RG][4];
#pragma unroll
  for (int j = 0; j < RG; ++j) {
    int mem, qh;
    column(j, mem, qh);
    const char* qrow = p.q + (int64_t(mem) * p.num_q_heads + qh) * ROWB;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) qb[j][kt] = *reinterpret_cast<const u32x4*>(qrow + 64 * kt + 16 * g);
  }
  // waves whose columns all lie past the set only stage
  const bool active = (RG * wave) * 16 < cols;

  // ---- staging: global -> registers -> LDS ----------------------------------
  const int32_t* trow = p.block_tables + int64_t(rep) * p.table_stride;
  const int64_t blk_stride = int64_t(p.num_kv_heads) * TILE;
  const char* kbase = p.k_cache + int64_t(kvh) * TILE;
  const char* vbase = p.v_cache + int64_t(kvh) * TILE;
  // table entries b0 + 64 c .. + 63 in one register, one per lane
  int tbl = -1, tbl_base = -kWave;
  auto table_entry = [&](int b) __attribute__((always_inline)) -> int {
    b = __builtin_amdgcn_readfirstlane(b);
    const int base = b0 + ((b - b0) & ~(kWave - 1));
    if (base != tbl_base) {  // wave-uniform; stages advance monotonically
      tbl_base = base;
      tbl = base + lane < b1 ? trow[base + lane] : -1;
    }
    return __builtin_amdgcn_readlane(tbl, b - base);
  };
  auto tile_rsrc = [&](const char* base, int blk) __attribute__((always_inline)) {
    const bool ok = unsigned(blk) < unsigned(p.num_blocks);
    return make_rsrc(base + (ok ? int64_t(blk) * blk_stride : 0), ok ? TILE : 0);
  };
  u32x4 kr[KL], vr0, vr1;
  bool bad_ld[2] = {false, false}, bad_c[2] = {false, false};
  auto load_stage = [&](int st) __attribute__((always_inline)) {
    int ids[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int j = b0 + 2 * st + b;
      ids[b] = j < b1 ? table_entry(j) : -1;
      bad_ld[b] = !(unsigned(ids[b]) < unsigned(p.num_blocks));
    }
#pragma unroll
    for (int i = 0; i < KL; ++i) {  // K: thread tid, token 16 i + tid / 16, chunk tid % 16
      const int tok = (tid + 256 * i) / CH, ch = tid % CH;
      kr[i] = load_tile<CP>(tile_rsrc(kbase, ids[i]), (tok % kBlockTokens) * ROWB + ch * 16);
    }
    {  // V: thread tid, tokens 2 (tid / 16) and the next, chunk tid % 16
      const int ch = tid % CH, tok = 2 * (tid / CH);
      const auto rs = tile_rsrc(vbase, ids[tok / kBlockTokens]);
      const int off = (tok % kBlockTokens) * ROWB + ch * 16;
      vr0 = load_tile<CP>(rs, off);
      vr1 = load_tile<CP>(rs, off + ROWB);
    }
  };
  auto store_stage = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int tok = (tid + 256 * i) / CH, ch = tid % CH;
      *reinterpret_cast<u32x4*>(&lk[buf][tok * KROW + ch * 8]) = kr[i];
    }
    const int ch = tid % CH, tok = 2 * (tid / CH);
    const uint32_t a[4] = {vr0.x, vr0.y, vr0.z, vr0.w};
    const uint32_t b[4] = {vr1.x, vr1.y, vr1.z, vr1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // Element e of token tok (low half) and of token tok + 1 (high half).
      const uint32_t w = __builtin_amdgcn_perm(b[e >> 1], a[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
      *reinterpret_cast<uint32_t*>(&lv[buf][(ch * 8 + e) * VROW + vt_col(ch * 8 + e, tok)]) = w;
    }
  };

  // ---- compute ----------------------------------------------------------------
  float m[RG], lsum[RG];
  f4 o[RG][NDT];
#pragma unroll
  for (int j = 0; j < RG; ++j) {
    m[j] = kNegBig;
    lsum[j] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[j][dt] = f4{0.f, 0.f, 0.f, 0.f};
  }
  auto compute = [&](int buf) __attribute__((always_inline)) {
    f4 sa[RG][2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int j = 0; j < RG; ++j) sa[j][blk] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&lk[buf][(blk * 16 + n) * KROW + 32 * kt + 8 * g]);
#pragma unroll
        for (int j = 0; j < RG; ++j) sa[j][blk] = mfma_k32<DT>(a, qb[j][kt], sa[j][blk]);
      }
    }
    const bool bad[2] = {bad_c[0], bad_c[1]};
    u32x4 pb[RG], pl[RG];
    float s[RG][8], mxl[RG];
    bool moved = false;
#pragma unroll
    for (int j = 0; j < RG; ++j) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int v = 0; v < 4; ++v) s[j][blk * 4 + v] = bad[blk] ? -INFINITY : sa[j][blk][v];
      mxl[j] = s[j][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mxl[j] = fmaxf(mxl[j], s[j][i]);
      // the lane's own scores decide whether any of the column's can move
      // its maximum; the column's maximum over its four lanes is formed
      // only in such a stage
      moved |= mxl[j] * c2 > m[j] + kSharedSlack;
    }
    float alpha[RG] = {};
#pragma unroll
    for (int j = 0; j < RG; ++j) alpha[j] = 1.f;
    bool rescale = false;
    if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
      for (int j = 0; j < RG; ++j) {
        const float mxs = max_over_lane_groups(mxl[j]) * c2;
        const float mn = mxs > m[j] + kSharedSlack ? mxs : m[j];
        alpha[j] = __builtin_amdgcn_exp2f(m[j] - mn);
        rescale |= mn > m[j];
        m[j] = mn;
      }
    }
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      const float mn = m[j];
      uint32_t ph[4], plo[4];
      float psum = 0.f;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j][2 * q2], c2, -mn));
        const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j][2 * q2 + 1], c2, -mn));
        const f2 xx = {x0, x1};
        if constexpr (DT == PKV_F16) {
          // the normaliser sums the weights as rounded (one dot product per pair)
          const h2 hp = __builtin_convertvector(xx, h2);
          ph[q2] = __builtin_bit_cast(uint32_t, hp);
          psum = __builtin_amdgcn_fdot2(hp, h2{1.f16, 1.f16}, psum, false);
        } else {
          psum += x0 + x1;
          const b2 hi2 = __builtin_convertvector(xx, b2);
          ph[q2] = __builtin_bit_cast(uint32_t, hi2);
          plo[q2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(xx - __builtin_convertvector(hi2, f2), b2));
        }
      }
      lsum[j] = lsum[j] * alpha[j] + psum;
      pb[j] = u32x4{ph[0], ph[1], ph[2], ph[3]};
      if constexpr (DT == PKV_BF16) pl[j] = u32x4{plo[0], plo[1], plo[2], plo[3]};
    }
    // rescale the accumulators only when some column's maximum moved
    if (__builtin_amdgcn_ballot_w64(rescale)) {
#pragma unroll
      for (int j = 0; j < RG; ++j)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[j][dt] *= alpha[j];
    }
    // V^T operands (dims 16 dt + n, tokens 4g .. 4g + 3 of each block),
    // each read one d-tile ahead of its products
    auto vt_operand = [&](int dt) __attribute__((always_inline)) -> u32x4 {
      const uint16_t* vrow = &lv[buf][(dt * 16 + n) * VROW];
      const u32x2 a0 = *reinterpret_cast<const u32x2*>(vrow + vt_col(dt * 16, 4 * g));
      const u32x2 a1 = *reinterpret_cast<const u32x2*>(vrow + vt_col(dt * 16, 16 + 4 * g));
      return u32x4{a0.x, a0.y, a1.x, a1.y};
    };
    u32x4 a_next = vt_operand(0);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const u32x4 a = a_next;
      if (dt + 1 < NDT) a_next = vt_operand(dt + 1);
#pragma unroll
      for (int j = 0; j < RG; ++j) {
        o[j][dt] = mfma_k32<DT>(a, pb[j], o[j][dt]);
        if constexpr (DT == PKV_BF16) o[j][dt] = mfma_k32<DT>(a, pl[j], o[j][dt]);
      }
    }
  };

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    const bool more = st + 1 < nst;
    bad_c[0] = bad_ld[0];
    bad_c[1] = bad_ld[1];
    if (more) load_stage(st + 1);
    if (active) compute(buf);
    if (more) store_stage(buf ^ 1);
    __syncthreads();
  }

  // records: column n of group j -> (member, query head) of the set
  const int64_t rec_step = int64_t(p.num_q_heads) * p.rec_floats;
#pragma unroll
  for (int j = 0; j < RG; ++j) {
    float lt = lsum[j] + __shfl_xor(lsum[j], 16);
    lt += __shfl_xor(lt, 32);
    int mem, qh;
    if (!column(j, mem, qh)) continue;
    const int po = p.part_offset[mem];
    const int ridx = po + k_base + chunk;
    if (po < 0 || ridx >= p.n_partials) continue;
    float* rec = p.part + int64_t(ridx) * rec_step + int64_t(qh) * p.rec_floats;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f4*>(rec + dt * 16 + 4 * g) = o[j][dt];
    if (g == 0) {
      rec[D] = m[j];
      rec[D + 1] = lt;
    }
  }
}

// Narrow shared nodes (at most 16 (member, query head) columns): one
// workgroup per (chunk, KV head) whose four waves stream the chunk's blocks
// as the grouped-query kernel does (register ping-pong, K through
// wave-private LDS rows into the A operand, V rows paired into the A
// operand of O^T += V^T P^T), with the node's columns as the 16 columns of
// the products.  The waves' states merge in LDS and become one record per
// column and chunk.  Blocks here are read once per launch: streaming loads.
template <int DT, int CP>
__global__ __launch_bounds__(256, 3) void paged_decode_narrow_kernel(const SharedParams p) {
  constexpr int NW = 4;
  constexpr int D = 128;
  constexpr int R = D * 2;
  constexpr int TILE = kBlockTokens * R;
  constexpr int KROWB = R + 16;
  __shared__ float sm_m[NW * 16];
  __shared__ float sm_l[NW * 16];
  __shared__ __attribute__((aligned(16))) float sm_o[NW * 16 * D];
  __shared__ __attribute__((aligned(16))) char sm_k[NW * kBlockTokens * KROWB];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane >> 4;
  const int n = lane & 15;
  const int item = blockIdx.x / p.num_kv_heads;
  const int kvh = blockIdx.x - item * p.num_kv_heads;
  int lo = 0, hi = p.n_nodes - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.nodes[kNodeInts * mid + 6] <= item) lo = mid;
    else hi = mid - 1;
  }
  const int32_t* nd = p.nodes + kNodeInts * lo;
  const int rep = nd[0], j0 = nd[1], j1 = nd[2], first = nd[3], members = nd[4], k_base = nd[5];
  const int chunk = item - nd[6];
  const int b0 = j0 + chunk * nd[8];
  const int b1 = min(j1, b0 + nd[8]);
  const int cols = min(16, members * p.group);
  const float c2 = p.scale_log2;
  char* const klds = sm_k + wave * kBlockTokens * KROWB;

  // column n: a (member, query head) pair of the node; past the node's
  // columns, copies of column 0 that write nothing
  auto column = [&](int c, int& mem, int& qh) __attribute__((always_inline)) {
    const int cc = c < cols ? c : 0;
    mem = p.order[first + cc / p.group];
    qh = kvh * p.group + (cc - (cc / p.group) * p.group);
  };
  u32x4 qb[4];
  {
    int mem, qh;
    column(n, mem, qh);
    const char* qrow = p.q + (int64_t(mem) * p.num_q_heads + qh) * R;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) qb[kc] = *reinterpret_cast<const u32x4*>(qrow + 64 * kc + 16 * g);
  }
  float m = kNegBig, lsum = 0.f;
  f4 o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = f4{0.f, 0.f, 0.f, 0.f};

  const int32_t* trow = p.block_tables + int64_t(rep) * p.table_stride;
  const int64_t blk_stride = int64_t(p.num_kv_heads) * TILE;
  int cb = 0, ce = 0, tbl = -1;
  const int koff = 16 * lane;
  const int voff = 4 * g * R + 16 * n;
  // every block of a node is full; a table entry outside the pool reads
  // nothing and is masked
  auto issue = [&](int j, u32x4* kk, u32x4* vv) __attribute__((always_inline)) -> bool {
    const int blk = __builtin_amdgcn_readlane(tbl, min(j - cb, kWave - 1));
    const bool ok = j < ce && unsigned(blk) < unsigned(p.num_blocks);
    const int64_t tile = int64_t(ok ? blk : 0) * blk_stride + int64_t(kvh) * TILE;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k_cache + tile, ok ? TILE : 0);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v_cache + tile, ok ? TILE : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) kk[i] = load_tile_s<CP>(rk, koff, 1024 * i);
#pragma unroll
    for (int t = 0; t < 4; ++t) vv[t] = load_tile_s<CP>(rv, voff, t * R);
    return ok;
  };
  auto process = [&](const u32x4* kk, const u32x4* vv, bool ok) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(klds + (4 * i + g) * KROWB + 16 * n) = kk[i];
    f4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
      sacc = mfma_k32<DT>(*reinterpret_cast<const u32x4*>(klds + n * KROWB + 64 * kc + 16 * g), qb[kc], sacc);
    float sc[4] = {sacc[0], sacc[1], sacc[2], sacc[3]};
    if (!ok) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = -INFINITY;
    }
    // as the matrix-core decode: the column's maximum lags by up to
    // kDecodeSlack and is exchanged across its lanes only when one lane's
    // scores pass it by more than that
    const float mxl = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    float alpha = 1.f;
    if (__builtin_amdgcn_ballot_w64(mxl * c2 > m + kDecodeSlack)) {
      const float mxs = max_over_lane_groups(mxl) * c2;
      const float mn = mxs > m + kDecodeSlack ? mxs : m;
      alpha = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
#pragma unroll
      for (int t = 0; t < 8; ++t) o[t] *= alpha;
    }
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], c2, -m));
    const f2 x01 = {x[0], x[1]}, x23 = {x[2], x[3]};
    u32x2 pb, pl;
    if constexpr (DT == PKV_F16) {
      // the normaliser sums the weights as rounded (one dot product per pair)
      const h2 h01 = __builtin_convertvector(x01, h2), h23 = __builtin_convertvector(x23, h2);
      pb = u32x2{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)};
      lsum = lsum * alpha + __builtin_amdgcn_fdot2(h23, h2{1.f16, 1.f16},
                                                   __builtin_amdgcn_fdot2(h01, h2{1.f16, 1.f16}, 0.f, false), false);
    } else {
      lsum = lsum * alpha + ((x[0] + x[1]) + (x[2] + x[3]));
      const b2 h01 = __builtin_convertvector(x01, b2), h23 = __builtin_convertvector(x23, b2);
      pb = u32x2{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)};
      pl = u32x2{__builtin_bit_cast(uint32_t, __builtin_convertvector(x01 - __builtin_convertvector(h01, f2), b2)),
                 __builtin_bit_cast(uint32_t, __builtin_convertvector(x23 - __builtin_convertvector(h23, f2), b2))};
    }
    const uint32_t v0[4] = {vv[0].x, vv[0].y, vv[0].z, vv[0].w};
    const uint32_t v1[4] = {vv[1].x, vv[1].y, vv[1].z, vv[1].w};
    const uint32_t v2[4] = {vv[2].x, vv[2].y, vv[2].z, vv[2].w};
    const uint32_t v3[4] = {vv[3].x, vv[3].y, vv[3].z, vv[3].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u32x2 lo2 = {(v0[w] & 0xFFFFu) | (v1[w] << 16), (v2[w] & 0xFFFFu) | (v3[w] << 16)};
      const u32x2 hi2 = {(v0[w] >> 16) | (v1[w] & 0xFFFF0000u), (v2[w] >> 16) | (v3[w] & 0xFFFF0000u)};
      o[2 * w] = mfma_k16<DT>(lo2, pb, o[2 * w]);
      o[2 * w + 1] = mfma_k16<DT>(hi2, pb, o[2 * w + 1]);
      if constexpr (DT == PKV_BF16) {
        o[2 * w] = mfma_k16<DT>(lo2, pl, o[2 * w]);
        o[2 * w + 1] = mfma_k16<DT>(hi2, pl, o[2 * w + 1]);
      }
    }
  };

  u32x4 ka[4], va[4], kb[4], vb[4];
  for (cb = b0; cb < b1; cb += kWave) {
    ce = min(cb + kWave, b1);
    tbl = (cb + lane < ce) ? trow[cb + lane] : -1;
    int j = cb + wave;
    if (j >= ce) break;
    bool ok_a = issue(j, ka, va), ok_b;
    while (true) {
      ok_b = issue(j + NW, kb, vb);
      process(ka, va, ok_a);
      j += NW;
      if (j >= ce) break;
      ok_a = issue(j + NW, ka, va);
      process(kb, vb, ok_b);
      j += NW;
      if (j >= ce) break;
    }
  }

  float lt = lsum + __shfl_xor(lsum, 16);
  lt += __shfl_xor(lt, 32);
  if (g == 0) {
    sm_m[wave * 16 + n] = m;
    sm_l[wave * 16 + n] = lt;
  }
  {
    float* orow = sm_o + (wave * 16 + n) * D + 32 * g;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *reinterpret_cast<f4*>(orow + 8 * r) = f4{o[0][r], o[1][r], o[2][r], o[3][r]};
      *reinterpret_cast<f4*>(orow + 8 * r + 4) = f4{o[4][r], o[5][r], o[6][r], o[7][r]};
    }
  }
  __syncthreads();
  const int64_t rec_step = int64_t(p.num_q_heads) * p.rec_floats;
  for (int idx = threadIdx.x; idx < cols * D; idx += 256) {
    const int c = idx / D;
    const int dd = idx - c * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w * 16 + c]);
    const float M_use = (M == -INFINITY) ? 0.f : M;
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = __builtin_amdgcn_exp2f(sm_m[w * 16 + c] - M_use);
      num = __builtin_fmaf(wt, sm_o[(w * 16 + c) * D + dd], num);
      den = __builtin_fmaf(wt, sm_l[w * 16 + c], den);
    }
    int mem, qh;
    column(c, mem, qh);
    const int po = p.part_offset[mem];
    const int ridx = po + k_base + chunk;
    if (po < 0 || ridx >= p.n_partials) continue;
    float* rec = p.part + int64_t(ridx) * rec_step + int64_t(qh) * p.rec_floats;
    rec[dd] = num;
    if (dd == 0) {
      rec[D] = M;
      rec[D + 1] = den;
    }
  }
}

struct ReduceParams {
  float* out;
  const float* part;
  const int32_t* context_lens;
  const int32_t* part_offset;
  const int32_t* reduce_seqs;
  const int32_t* priv_start;  // or null
  const int32_t* n_shared;    // or null
  int32_t num_q_heads;
  int32_t table_stride;
  int32_t partition_blocks;
  int32_t n_partials;
  int32_t rec_floats;
};

// Separate combine kernel (two-launch variant): one workgroup of D threads
// per (multi-partition sequence, query head).
template <int D>
__global__ __launch_bounds__(D) void paged_decode_reduce_kernel(const ReduceParams p) {
  const int r = blockIdx.x / p.num_q_heads;
  const int h = blockIdx.x - r * p.num_q_heads;
  const int seq = p.reduce_seqs[r];
  const int L = p.context_lens[seq];
  const int nblk = min((L + kBlockTokens - 1) / kBlockTokens, p.table_stride);
  const int ps = p.priv_start ? p.priv_start[seq] : 0;
  const int n_parts = (p.n_shared ? p.n_shared[seq] : 0) + (nblk - ps + p.partition_blocks - 1) / p.partition_blocks;
  const int base = p.part_offset[seq];
  if (base < 0 || base + n_parts > p.n_partials) return;
  const int dd = threadIdx.x;
  const float* rec0 = p.part + (int64_t(base) * p.num_q_heads + h) * p.rec_floats;
  const int64_t step = int64_t(p.num_q_heads) * p.rec_floats;
  float M = -INFINITY, num = 0.f, den = 0.f;
  merge_records<D, false>(rec0, step, n_parts, dd, M, num, den);
  p.out[(int64_t(seq) * p.num_q_heads + h) * D + dd] = num / den;
}

using DecodeFn = void (*)(const DecodeParams);

// The pickers take the requested waves per workgroup in nw and leave there
// the waves of the instance they return (an instance may not exist for every
// request): the launch's block size must be that instance's.  With `reuse`
// (a batch that shares blocks) they return the 4-wave instance with cached
// tile loads whatever the request.
// PKV_DECODE_LDS_PAD=<bytes> adds that much unused dynamic LDS to every
// workgroup of the decode launch, capping how many workgroups a CU holds:
// a tuning variable for occupancy sweeps, read at every launch (0 to 64 KiB;
// pkv_decode_occupancy does not see it).
size_t lds_pad_bytes() {
  const char* s = std::getenv("PKV_DECODE_LDS_PAD");
  const long v = s ? std::atol(s) : 0;
  return v > 0 && v <= 65536 ? size_t(v) : 0;
}

// The VALU kernel of fp16 / bf16, head_dim 128, one query head per
// workgroup and four waves stages its tiles through LDS: on MI355X that
// instance decodes the GPT-style fp16 batch (64 sequences, 32 heads) in
// 72.4 us against 74.4 us for register staging at the same two or three
// workgroups per CU, and the long bf16 batch in the same time.
// PKV_DECODE_STAGING=regs selects the register-staged instance instead, for
// comparisons; read at every launch.
bool lds_staging() {
  const char* s = std::getenv("PKV_DECODE_STAGING");
  return !(s && std::string(s) == "regs");
}

template <int DT, int D, int GW>
DecodeFn pick_waves(int& nw, bool reuse) {
  if (reuse) {
    nw = 4;
    return paged_decode_kernel<DT, D, GW, 4, kCacheReuse>;
  }
  if constexpr (GW == 1 && D == 128 && DT != PKV_F32) {
    if (nw == 4 && lds_staging()) return paged_decode_kernel<DT, D, GW, 4, kCacheStream, true>;
  }
  switch (nw) {
    case 1: return paged_decode_kernel<DT, D, GW, 1>;
    case 2: return paged_decode_kernel<DT, D, GW, 2>;
    case 4: return paged_decode_kernel<DT, D, GW, 4>;
    case 8:  // 512 threads; its LDS merge area fits 64 KiB for GW <= 2 only
      if constexpr (GW <= 2) return paged_decode_kernel<DT, D, GW, 8>;
      nw = 4;
      return paged_decode_kernel<DT, D, GW, 4>;
    default: return nullptr;
  }
}

template <int DT, int D>
DecodeFn pick_gw(int gw, int& nw, bool reuse) {
  switch (gw) {
    case 1: return pick_waves<DT, D, 1>(nw, reuse);
    case 2: return pick_waves<DT, D, 2>(nw, reuse);
    case 4: return pick_waves<DT, D, 4>(nw, reuse);
    case 8: return pick_waves<DT, D, 8>(nw, reuse);
    default: return nullptr;
  }
}

template <int DT>
DecodeFn pick_d(int d, int gw, int& nw, bool reuse) {
  switch (d) {
    case 64: return pick_gw<DT, 64>(gw, nw, reuse);
    case 128: return pick_gw<DT, 128>(gw, nw, reuse);
    case 256: return pick_gw<DT, 256>(gw, nw, reuse);
    default: return nullptr;
  }
}

DecodeFn pick_decode(int dt, int d, int gw, int& nw, bool reuse) {
  switch (dt) {
    case PKV_F32: return pick_d<PKV_F32>(d, gw, nw, reuse);
    case PKV_F16: return pick_d<PKV_F16>(d, gw, nw, reuse);
    case PKV_BF16: return pick_d<PKV_BF16>(d, gw, nw, reuse);
    default: return nullptr;
  }
}

template <int DT, int GW>
DecodeFn pick_mfma_waves(int& nw, bool reuse) {
  if (reuse) {
    nw = 4;
    return paged_decode_mfma_kernel<DT, GW, 4, kCacheReuse>;
  }
  switch (nw) {
    case 1: return paged_decode_mfma_kernel<DT, GW, 1>;
    case 2: return paged_decode_mfma_kernel<DT, GW, 2>;
    case 4: return paged_decode_mfma_kernel<DT, GW, 4>;
    case 8:  // its LDS merge area fits 32 KiB for GW <= 8
      if constexpr (GW <= 8) return paged_decode_mfma_kernel<DT, GW, 8>;
      nw = 4;
      return paged_decode_mfma_kernel<DT, GW, 4>;
    default: return nullptr;
  }
}

template <int DT>
DecodeFn pick_mfma_gw(int gw, int& nw, bool reuse) {
  switch (gw) {
    case 2: return pick_mfma_waves<DT, 2>(nw, reuse);
    case 4: return pick_mfma_waves<DT, 4>(nw, reuse);
    case 8: return pick_mfma_waves<DT, 8>(nw, reuse);
    case 16: return pick_mfma_waves<DT, 16>(nw, reuse);
    default: return nullptr;
  }
}

DecodeFn pick_mfma(int dt, int gw, int& nw, bool reuse) {
  switch (dt) {
    case PKV_F16: return pick_mfma_gw<PKV_F16>(gw, nw, reuse);
    case PKV_BF16: return pick_mfma_gw<PKV_BF16>(gw, nw, reuse);
    default: return nullptr;
  }
}

// Waves per workgroup (they split a work item's blocks): 4 for items of 16
// blocks or more on average (the best of {1, 2, 4, 8} on the GPT-style fp16
// batch, ~28 blocks per item), 2 from 6 blocks and 1 below: a short item
// leaves most of four waves idle.  The own parts that follow shared-block
// launches take one wave whatever their length: each also merges its
// sequence's shared records, and more, smaller workgroups finish sooner (a
// prefix-shared batch of 256 over its 56 timed iterations, own parts of 3 to
// ~17 blocks on average: 0.2134-0.2140 ms per decode with one wave against
// 0.2160-0.2175 with the length rule).
// PKV_DECODE_WAVES overrides the choice for tuning sweeps.  The tuning
// variables are read at every launch (a lookup in the environment, next to
// a launch of tens of microseconds), so one process can run every variant.
int waves_per_item(int item_blocks, bool after_shared = false) {
  const char* s = std::getenv("PKV_DECODE_WAVES");
  const int v = s ? std::atoi(s) : 0;
  if (v == 1 || v == 2 || v == 4 || v == 8) return v;
  if (after_shared) return 1;
  return item_blocks >= 16 ? 4 : item_blocks >= 6 ? 2 : 1;
}

// Query heads of one KV head that one workgroup takes (GW): all of them,
// up to 8 on the VALU kernel and 16 on the matrix-core one.  Splitting a KV
// head's query heads over workgroups makes each read the tiles (the
// nontemporal loads keep no copy in L2 for the others; measured 1.45x
// slower for GQA-4 split in two).  PKV_DECODE_GW caps it for tuning sweeps.
int heads_per_workgroup(int group, int limit) {
  const char* s = std::getenv("PKV_DECODE_GW");
  const int v = s ? std::atoi(s) : 0;
  const int cap = (v == 1 || v == 2 || v == 4 || v == 8 || v == 16) ? v : 16;
  limit = std::min(limit, cap);
  int gw = 1;
  while (gw < limit && group % (2 * gw) == 0) gw *= 2;
  return gw;
}

// Grouped-query batches of fp16 / bf16 with head_dim 128 run on the
// matrix-core kernel when at least two query heads share a workgroup.
// PKV_DECODE_MFMA=0 selects the VALU kernel instead; it is read at every
// launch, so one process can run and compare both.
bool mfma_eligible(int group, int32_t dtype, int32_t head_dim) {
  if (group < 2 || head_dim != 128 || (dtype != PKV_F16 && dtype != PKV_BF16)) return false;
  const char* s = std::getenv("PKV_DECODE_MFMA");
  return !(s && s[0] == '0');
}

// Validate the arguments shared by the decode entry points and fill the
// kernel parameters.  Returns PKV_OK with *empty set when there is no work.
pkv_status setup_decode(const pkv_pool* pool, const void* q, const void* k_new, const void* v_new,
                        float* out, int32_t num_seqs, int32_t num_q_heads,
                        const int32_t* block_tables, int32_t table_stride,
                        const int32_t* context_lens, float scale, const int32_t* plan,
                        const pkv_decode_plan_info* info, void* workspace, size_t workspace_bytes,
                        DecodeParams& prm, int& gw, bool& mfma, bool& empty) {
  empty = false;
  if (!pool) return fail(PKV_E_BAD_ARG, "null pool");
  const pkv_pool_desc& d = pool->desc;
  if (!pool->k_cache || !pool->v_cache) return fail(PKV_E_BAD_ARG, "pool has no device K/V arrays");
  if (d.block_size != kBlockTokens)
    return fail(PKV_E_UNSUPPORTED, "device kernels take block_size 16 only");
  if (d.head_dim != 64 && d.head_dim != 128 && d.head_dim != 256)
    return fail(PKV_E_UNSUPPORTED, "head_dim must be 64, 128 or 256");
  if (!info) return fail(PKV_E_BAD_ARG, "null plan info");
  // the matrix-core kernel scales a block's maximum score after taking it,
  // which equals the maximum of the scaled scores only for a positive scale
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(PKV_E_BAD_ARG, "scale must be finite and > 0");
  if (num_seqs < 0 || num_q_heads < 1 || num_q_heads % d.num_kv_heads != 0)
    return fail(PKV_E_BAD_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  if (info->num_seqs != num_seqs || info->block_size != d.block_size ||
      info->partition_tokens < kBlockTokens || info->partition_tokens % kBlockTokens != 0 ||
      info->n_work < 0 || info->n_partials < 0 || info->n_reduce < 0)
    return fail(PKV_E_BAD_ARG, "plan info does not match this batch");
  if (table_stride < 1) return fail(PKV_E_BAD_ARG, "table_stride must be >= 1");
  if (int64_t(info->max_context_len) > int64_t(table_stride) * kBlockTokens)
    return fail(PKV_E_BAD_ARG, "a context is longer than its table can address");
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(PKV_E_BAD_ARG, "k_new and v_new must both be given or both be NULL");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
    return fail(PKV_E_BAD_ARG, "k_new and v_new must be 16-byte aligned");
  if (num_seqs == 0 || info->n_work == 0) {
    empty = true;
    return PKV_OK;
  }
  if (!q || !out || !block_tables || !context_lens || !plan)
    return fail(PKV_E_BAD_ARG, "null device pointer");
  const size_t need = pkv_decode_workspace_bytes(info, num_q_heads, d.head_dim);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PKV_E_BAD_ARG, "workspace too small: need " + std::to_string(need) + " bytes");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(workspace)) & 15 ||
      reinterpret_cast<uintptr_t>(out) & 3)
    return fail(PKV_E_BAD_ARG, "q and workspace must be 16-byte aligned and out 4-byte aligned");
  const int group = num_q_heads / d.num_kv_heads;
  mfma = mfma_eligible(group, d.dtype, d.head_dim);
  gw = heads_per_workgroup(group, mfma ? 16 : 8);
  if (gw < 2) mfma = false;
  prm.q = static_cast<const char*>(q);
  prm.k_new = static_cast<const char*>(k_new);
  prm.v_new = static_cast<const char*>(v_new);
  prm.out = out;
  prm.k_cache = static_cast<char*>(pool->k_cache);
  prm.v_cache = static_cast<char*>(pool->v_cache);
  prm.block_tables = block_tables;
  prm.context_lens = context_lens;
  prm.work = plan;
  prm.part_offset = plan + 2 * int64_t(info->n_work);
  prm.priv_start = nullptr;
  prm.n_shared = nullptr;
  if (info->n_nodes > 0) {
    if ((d.dtype != PKV_F16 && d.dtype != PKV_BF16) || d.head_dim != 128)
      return fail(PKV_E_UNSUPPORTED, "shared-block plans take fp16 / bf16 pools of head_dim 128");
    if (info->shared_group != group || info->shared_chunk_blocks < 1 || info->narrow_chunk_blocks < 1 ||
        info->n_wide_nodes < 0 || info->n_wide_nodes > info->n_nodes || info->n_shared_items < 0 ||
        info->n_narrow_items < 0 || info->off_shared < 2 * info->n_work + num_seqs + info->n_reduce ||
        int64_t(info->off_shared) + 3 * int64_t(num_seqs) + kNodeInts * int64_t(info->n_nodes) > info->plan_ints)
      return fail(PKV_E_BAD_ARG, "shared-block plan does not match this batch (made for another head count?)");
    if (int64_t(std::max(info->n_shared_items, info->n_narrow_items)) * d.num_kv_heads > INT32_MAX)
      return fail(PKV_E_BAD_ARG, "shared launch too large");
    prm.priv_start = plan + info->off_shared;
    prm.n_shared = prm.priv_start + num_seqs;
  }
  // workspace: records from its start, one per (partial, query head):
  // o[D], m, l padded to 128 bytes; completion tickets [num_seqs][H_q] at
  // its end (128-byte aligned).  A workspace shared by launches of
  // different shapes and sized for the largest (pkv_decode_workspace_bound)
  // therefore never has one launch's records where another's tickets are.
  char* ws = static_cast<char*>(workspace);
  const int64_t ticket_bytes = (int64_t(num_seqs) * num_q_heads * 4 + 255) / 256 * 256;
  prm.part = reinterpret_cast<float*>(ws);
  prm.counters = reinterpret_cast<int32_t*>(
      ws + ((int64_t(workspace_bytes) - ticket_bytes) & ~int64_t(127)));
  prm.rec_floats = int32_t(((int64_t(d.head_dim) + 2) * 4 + 127) / 128 * 32);
  prm.num_q_heads = num_q_heads;
  prm.num_kv_heads = d.num_kv_heads;
  prm.group = group;
  prm.hgroups_per_kv = group / gw;
  prm.table_stride = table_stride;
  prm.num_blocks = d.num_blocks;
  prm.partition_blocks = info->partition_tokens / kBlockTokens;
  prm.n_partials = info->n_partials;
  prm.scale_log2 = scale * kLog2e;
  if (int64_t(info->n_work) * d.num_kv_heads * prm.hgroups_per_kv > INT32_MAX ||
      int64_t(info->n_reduce) * num_q_heads > INT32_MAX)
    return fail(PKV_E_BAD_ARG, "batch too large for one launch");
  return PKV_OK;
}

// A second stream per device for the narrow shared-block launch, so that it
// runs beside the wide one: the wide kernel is bound by its matrix-core
// chain at two workgroups per CU and leaves registers and LDS for one
// narrow workgroup on each CU.  Created on the first such call on the
// device; the fork / join events are recorded and waited for under a lock,
// so that calls from several host threads keep their own dependencies.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kSideDevices = 64;
std::mutex side_mu;
SideStream side_tab[kSideDevices];

// *out stays null when the side stream does not exist yet and `s` is being
// captured into a graph (nothing is created during a capture).
pkv_status side_stream(hipStream_t s, SideStream** out) {  // caller holds side_mu
  *out = nullptr;
  // the device of the caller's stream (the current one for the null stream)
  int cur = -1, dev = -1;
  if (hipGetDevice(&cur) != hipSuccess) return launch_status("current device query");
  if (s == nullptr) dev = cur;
  else if (hipStreamGetDevice(s, &dev) != hipSuccess) return launch_status("stream device query");
  if (dev < 0 || dev >= kSideDevices) return fail(PKV_E_HIP, "device out of range for the shared-block side stream");
  SideStream& ss = side_tab[dev];
  if (!ss.stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return launch_status("stream capture query");
    if (cs != hipStreamCaptureStatusNone) return PKV_OK;
    // created on the stream's device, the current device restored after
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return launch_status("side stream device");
    SideStream n;
    const bool ok = hipStreamCreateWithFlags(&n.stream, hipStreamNonBlocking) == hipSuccess &&
                    hipEventCreateWithFlags(&n.fork, hipEventDisableTiming) == hipSuccess &&
                    hipEventCreateWithFlags(&n.join, hipEventDisableTiming) == hipSuccess;
    if (!ok) {  // nothing half made is kept
      if (n.join) (void)hipEventDestroy(n.join);
      if (n.fork) (void)hipEventDestroy(n.fork);
      if (n.stream) (void)hipStreamDestroy(n.stream);
    } else {
      ss = n;
    }
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return launch_status("current device restore");
    if (!ok) return launch_status("shared-block side stream creation");
  }
  *out = &ss;
  return PKV_OK;
}

// ev_start / ev_stop (optional) are attached to the dispatch itself
// (hipExtLaunchKernel), so their interval is the kernel's execution, without
// the queueing of separate marker packets.
// The shared-block launches of a plan with nodes: one workgroup per (shared
// item, KV head), writing the nodes' split-K records; wide nodes on `s`,
// narrow ones on the side stream when `concurrent` (joined back into `s`),
// else after the wide launch on `s`.
pkv_status launch_shared(const pkv_pool* pool, const DecodeParams& prm, const int32_t* plan,
                         const pkv_decode_plan_info* info, hipStream_t s, hipEvent_t ev_start,
                         bool concurrent) {
  SharedParams sp;
  sp.q = prm.q;
  sp.k_cache = prm.k_cache;
  sp.v_cache = prm.v_cache;
  sp.block_tables = prm.block_tables;
  sp.part_offset = prm.part_offset;
  sp.order = plan + info->off_shared + 2 * int64_t(info->num_seqs);
  sp.nodes = sp.order + info->num_seqs;
  sp.part = prm.part;
  sp.rec_floats = prm.rec_floats;
  sp.num_q_heads = prm.num_q_heads;
  sp.num_kv_heads = prm.num_kv_heads;
  sp.group = prm.group;
  sp.table_stride = prm.table_stride;
  sp.num_blocks = prm.num_blocks;
  sp.n_nodes = info->n_wide_nodes;
  sp.per_set = kSharedCols / prm.group;
  sp.n_partials = info->n_partials;
  sp.scale_log2 = prm.scale_log2;
  // PKV_SHARED_WAVES (2 or 3, read at every launch) picks the register
  // budget for tuning sweeps
  const char* e = std::getenv("PKV_SHARED_WAVES");
  const bool three = e && e[0] == '3';
  void (*fn)(const SharedParams) =
      pool->desc.dtype == PKV_F16
          ? (three ? paged_decode_shared_kernel<PKV_F16, kCacheReuse, 3> : paged_decode_shared_kernel<PKV_F16, kCacheReuse, 2>)
          : (three ? paged_decode_shared_kernel<PKV_BF16, kCacheReuse, 3> : paged_decode_shared_kernel<PKV_BF16, kCacheReuse, 2>);
  const bool wide = info->n_wide_nodes > 0 && info->n_shared_items > 0;
  const bool narrow = info->n_nodes > info->n_wide_nodes && info->n_narrow_items > 0;
  SharedParams np = sp;
  np.nodes = sp.nodes + kNodeInts * int64_t(info->n_wide_nodes);
  np.n_nodes = info->n_nodes - info->n_wide_nodes;
  void (*nfn)(const SharedParams) = pool->desc.dtype == PKV_F16 ? paged_decode_narrow_kernel<PKV_F16, kCacheStream>
                                                                : paged_decode_narrow_kernel<PKV_BF16, kCacheStream>;
  const uint32_t wgrid = uint32_t(int64_t(info->n_shared_items) * prm.num_kv_heads);
  const uint32_t ngrid = uint32_t(int64_t(info->n_narrow_items) * prm.num_kv_heads);
  // PKV_SHARED_CONCURRENT=0 (read at every launch) keeps both on `s`
  const char* ce = std::getenv("PKV_SHARED_CONCURRENT");
  std::unique_lock<std::mutex> lock(side_mu, std::defer_lock);
  SideStream* ss = nullptr;
  if (wide && narrow && concurrent && !(ce && ce[0] == '0')) {
    lock.lock();
    if (pkv_status st = side_stream(s, &ss)) return st;
  }
  if (ss) {
    // a start event brackets both launches from here
    if (ev_start && hipEventRecord(ev_start, s) != hipSuccess) return launch_status("decode start event");
    if (hipEventRecord(ss->fork, s) != hipSuccess || hipStreamWaitEvent(ss->stream, ss->fork, 0) != hipSuccess)
      return launch_status("shared-block fork");
    hipLaunchKernelGGL(nfn, dim3(ngrid), dim3(256), 0, ss->stream, np);
    if (pkv_status st = launch_status("paged_decode narrow shared-block launch")) return st;
    if (hipEventRecord(ss->join, ss->stream) != hipSuccess) return launch_status("shared-block join record");
    hipLaunchKernelGGL(fn, dim3(wgrid), dim3(256), 0, s, sp);
    if (pkv_status st = launch_status("paged_decode wide shared-block launch")) return st;
    if (hipStreamWaitEvent(s, ss->join, 0) != hipSuccess) return launch_status("shared-block join");
    return PKV_OK;
  }
  if (wide) {
    if (ev_start)
      hipExtLaunchKernelGGL(fn, dim3(wgrid), dim3(256), 0, s, ev_start, nullptr, 0, sp);
    else
      hipLaunchKernelGGL(fn, dim3(wgrid), dim3(256), 0, s, sp);
    if (pkv_status st = launch_status("paged_decode wide shared-block launch")) return st;
    ev_start = nullptr;
  }
  if (narrow) {
    if (ev_start)
      hipExtLaunchKernelGGL(nfn, dim3(ngrid), dim3(256), 0, s, ev_start, nullptr, 0, np);
    else
      hipLaunchKernelGGL(nfn, dim3(ngrid), dim3(256), 0, s, np);
    if (pkv_status st = launch_status("paged_decode narrow shared-block launch")) return st;
  }
  return PKV_OK;
}

// concurrent: the narrow shared-block launch may run on the side stream
// (not for the no-allocation entry point, which creates nothing)
pkv_status launch_partitions(const pkv_pool* pool, const DecodeParams& prm, int gw, bool mfma,
                             const pkv_decode_plan_info* info, hipStream_t s,
                             hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr,
                             bool concurrent = true) {
  if (info->n_nodes > 0) {
    // blocks held in common first: their records must exist before the
    // decode launch below combines them (stream order, or the join)
    if (pkv_status st = launch_shared(pool, prm, prm.work, info, s, ev_start, concurrent)) return st;
    ev_start = nullptr;
  }
  int nw = waves_per_item(info->item_blocks, info->n_nodes > 0);  // becomes the chosen instance's waves
  const bool reuse = info->shared_kv != 0;
  DecodeFn fn = mfma ? pick_mfma(pool->desc.dtype, gw, nw, reuse)
                     : pick_decode(pool->desc.dtype, pool->desc.head_dim, gw, nw, reuse);
  if (!fn) return fail(PKV_E_UNSUPPORTED, "no kernel for this dtype / head_dim / group");
  const int64_t grid = int64_t(info->n_work) * prm.num_kv_heads * prm.hgroups_per_kv;
  const size_t pad = lds_pad_bytes();
  if (ev_start || ev_stop)  // one start / stop pair spans both launches of a shared-block plan
    hipExtLaunchKernelGGL(fn, dim3(uint32_t(grid)), dim3(kWave * nw), pad, s, ev_start, ev_stop, 0, prm);
  else
    hipLaunchKernelGGL(fn, dim3(uint32_t(grid)), dim3(kWave * nw), pad, s, prm);
  return launch_status("paged_decode launch");
}

pkv_status launch_reduce(const pkv_pool* pool, const DecodeParams& prm, int32_t num_seqs,
                         const pkv_decode_plan_info* info, hipStream_t s) {
  if (info->n_reduce == 0) return PKV_OK;
  ReduceParams rp;
  rp.out = prm.out;
  rp.part = prm.part;
  rp.rec_floats = prm.rec_floats;
  rp.context_lens = prm.context_lens;
  rp.part_offset = prm.part_offset;
  rp.reduce_seqs = prm.part_offset + num_seqs;
  rp.priv_start = prm.priv_start;
  rp.n_shared = prm.n_shared;
  rp.num_q_heads = prm.num_q_heads;
  rp.table_stride = prm.table_stride;
  rp.partition_blocks = prm.partition_blocks;
  rp.n_partials = info->n_partials;
  void (*rfn)(const ReduceParams) = nullptr;
  switch (pool->desc.head_dim) {
    case 64: rfn = paged_decode_reduce_kernel<64>; break;
    case 128: rfn = paged_decode_reduce_kernel<128>; break;
    case 256: rfn = paged_decode_reduce_kernel<256>; break;
  }
  const int64_t rgrid = int64_t(info->n_reduce) * prm.num_q_heads;
  hipLaunchKernelGGL(rfn, dim3(uint32_t(rgrid)), dim3(pool->desc.head_dim), 0, s, rp);
  return launch_status("paged_decode_reduce launch");
}

}  // namespace
}  // namespace pkv

using namespace pkv;

#define PKV_SETUP                                                                                \
  DecodeParams prm;                                                                              \
  int gw = 1;                                                                                    \
  bool mfma = false, empty = false;                                                              \
  if (pkv_status st = setup_decode(pool, q, k_new, v_new, out, num_seqs, num_q_heads,           \
                                   block_tables, table_stride, context_lens, scale, plan, info, \
                                   workspace, workspace_bytes, prm, gw, mfma, empty))           \
    return st;                                                                                   \
  if (empty) return PKV_OK;                                                                      \
  hipStream_t s = static_cast<hipStream_t>(stream);

extern "C" pkv_status pkv_decode_occupancy(const pkv_pool* pool, int32_t num_q_heads,
                                           int32_t* workgroups_per_item, int64_t* resident) {
  if (!pool || !workgroups_per_item || !resident) return fail(PKV_E_BAD_ARG, "null pool or output");
  const pkv_pool_desc& d = pool->desc;
  if (num_q_heads < 1 || num_q_heads % d.num_kv_heads != 0)
    return fail(PKV_E_BAD_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  const int group = num_q_heads / d.num_kv_heads;
  bool mfma = mfma_eligible(group, d.dtype, d.head_dim);
  const int gw = heads_per_workgroup(group, mfma ? 16 : 8);
  if (gw < 2) mfma = false;
  int nw = waves_per_item(16);  // long items, where filling the GPU matters; becomes the instance's waves
  DecodeFn fn = mfma ? pick_mfma(d.dtype, gw, nw, false) : pick_decode(d.dtype, d.head_dim, gw, nw, false);
  if (!fn) return fail(PKV_E_UNSUPPORTED, "no kernel for this dtype / head_dim / group");
  int per_cu = 0, dev = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), kWave * nw, 0) !=
          hipSuccess ||
      hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return launch_status("decode occupancy query");
  *workgroups_per_item = d.num_kv_heads * (group / gw);
  *resident = int64_t(per_cu) * cus;
  return PKV_OK;
}

extern "C" pkv_status pkv_paged_decode(PKV_DECODE_ARGS) {
  PKV_SETUP
  return launch_partitions(pool, prm, gw, mfma, info, s);  // combine fused in
}

pkv_status pkv::paged_decode_timed(PKV_DECODE_ARGS, hipEvent_t ev_start, hipEvent_t ev_stop) {
  PKV_SETUP
  return launch_partitions(pool, prm, gw, mfma, info, s, ev_start, ev_stop);
}

extern "C" pkv_status pkv_paged_decode_partitions(PKV_DECODE_ARGS) {
  PKV_SETUP
  prm.counters = nullptr;  // partials only; pkv_paged_decode_reduce combines
  return launch_partitions(pool, prm, gw, mfma, info, s);
}

extern "C" pkv_status pkv_paged_decode_reduce(PKV_DECODE_ARGS) {
  PKV_SETUP
  (void)gw;
  (void)mfma;
  return launch_reduce(pool, prm, num_seqs, info, s);
}

// ---------------------------------------------------------------------------
// Decode without a caller workspace, for callers that cannot allocate device
// memory.  Its split-K records and completion tickets live in `scratch`, a
// fixed array of this library's code object: every GPU the library runs on
// holds one copy of PKV_NOALLOC_SCRATCH_BYTES until the process ends.  In
// host code the array's name only stands for the device symbol; its device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current and kept in scratch_ptr.  Calls on one device share the
// array: calls that overlap in time on one GPU race.
static __device__ __align__(256) char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace pkv {
namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (set up on the first call
// on that device).
pkv_status current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(PKV_E_HIP, "no current HIP device for the decode scratch");
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PKV_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return PKV_OK;
}

// Zero n completion tickets (a plain kernel, not a memset node, so that the
// call stays valid inside a captured graph).
__global__ __launch_bounds__(256) void clear_tickets_kernel(int32_t* tickets, int n) {
  const int i = int(blockIdx.x) * 256 + int(threadIdx.x);
  if (i < n) tickets[i] = 0;
}

}  // namespace
}  // namespace pkv

extern "C" pkv_status pkv_paged_decode_noalloc(const pkv_pool* pool, const void* q, const void* k_new,
                                               const void* v_new, float* out, int32_t num_seqs,
                                               int32_t num_q_heads, const int32_t* block_tables,
                                               int32_t table_stride, const int32_t* context_lens,
                                               float scale, const int32_t* plan,
                                               const pkv_decode_plan_info* info, void* stream) {
  if (!pool || !info) return fail(PKV_E_BAD_ARG, "null pool or plan info");
  const size_t need = pkv_decode_workspace_bytes(info, num_q_heads, pool->desc.head_dim);
  if (need > size_t(PKV_NOALLOC_SCRATCH_BYTES))
    return fail(PKV_E_BAD_ARG, "this batch needs " + std::to_string(need) +
                                   " bytes of split-K scratch; the no-allocation decode holds " +
                                   std::to_string(size_t(PKV_NOALLOC_SCRATCH_BYTES)) +
                                   " (use pkv_paged_decode with a workspace, or longer partitions)");
  void* ws = nullptr;
  if (pkv_status st = current_scratch(&ws)) return st;
  const size_t workspace_bytes = size_t(PKV_NOALLOC_SCRATCH_BYTES);
  void* workspace = ws;
  PKV_SETUP
  if (info->n_reduce > 0) {
    // this launch's tickets start at zero whatever an earlier call left there
    const int n = num_seqs * num_q_heads;
    hipLaunchKernelGGL(clear_tickets_kernel, dim3(uint32_t((n + 255) / 256)), dim3(256), 0, s, prm.counters, n);
    if (pkv_status st = launch_status("decode scratch ticket clear")) return st;
  }
  return launch_partitions(pool, prm, gw, mfma, info, s, nullptr, nullptr, false);
}
