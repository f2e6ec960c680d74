// Gather probe: the K/V tile reads of a decode launch, with none of its
// arithmetic.
//
// A decode is bound by the rate at which it can gather (block, KV head)
// tiles through the block tables ("04 — Hacia PagedAttention", La idea de
// PagedAttention, step 5): each tile is 16 rows x R bytes, contiguous, at a
// place the table decides.  This kernel walks exactly the tiles a decode
// plan makes the decode read (same work items, same order, same partition
// bounds, K and V), with the same wave layout (one workgroup per work item
// and KV head, waves striding over the item's blocks, lane l taking bytes
// [16 l, 16 l + 16) of each 1 KiB of a tile), and folds every 32-bit word it
// loads into one XOR per wave so the loads cannot be dropped.  Its time is
// the gather ceiling the decode kernels are measured against; the staging
// modes show what each way of moving a tile costs on its own:
//   PKV_PROBE_REGS:   the tile goes to registers, two register sets
//                     alternate (the next block loads while the current one
//                     is folded), nontemporal loads;
//   PKV_PROBE_CACHED: the same with ordinary (cached) loads;
//   PKV_PROBE_LDS:    the tile goes straight to LDS (buffer loads with the
//                     LDS bit, no registers in flight), into a per-wave ring
//                     of two stages, and is read back from LDS to be folded;
//                     nontemporal loads.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"

namespace pkv {
namespace {

struct ProbeParams {
  const char* k_cache;
  const char* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* work;  // (sequence, partition) per item
  uint32_t* out;        // [n_work][num_kv_heads][NW]
  int32_t num_kv_heads;
  int32_t table_stride;
  int32_t num_blocks;
  int32_t partition_blocks;
  int32_t tile_bytes;
};

__device__ __forceinline__ uint32_t fold(const u32x4& v) { return v.x ^ v.y ^ v.z ^ v.w; }

template <int NI, int CP, int NW>
__global__ __launch_bounds__(kWave* NW) void gather_probe_kernel(const ProbeParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wi = blockIdx.x / p.num_kv_heads;
  const int kvh = blockIdx.x - wi * p.num_kv_heads;
  const int seq = p.work[2 * wi];
  const int part = p.work[2 * wi + 1];
  const int L = p.context_lens[seq];
  const int nblk = min((L + kBlockTokens - 1) / kBlockTokens, p.table_stride);
  const int b0 = part * p.partition_blocks;
  const int b1 = min(b0 + p.partition_blocks, nblk);
  const int32_t* trow = p.block_tables + int64_t(seq) * p.table_stride;
  const int TILE = p.tile_bytes;
  const int64_t blk_stride = int64_t(p.num_kv_heads) * TILE;

  // Block j of the current 64-entry table chunk [cb, ce): as in the decode,
  // the loads are always issued and a block past the chunk (or outside the
  // pool) gets a 0-record resource, which returns zeros and reads nothing.
  int cb = 0, ce = 0, tbl = -1;
  auto issue = [&](int j, u32x4* kk, u32x4* vv) __attribute__((always_inline)) {
    const int blk = __builtin_amdgcn_readlane(tbl, min(j - cb, kWave - 1));
    const bool ok = j < ce && unsigned(blk) < unsigned(p.num_blocks);
    const int64_t tile = int64_t(ok ? blk : 0) * blk_stride + int64_t(kvh) * TILE;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k_cache + tile, ok ? TILE : 0);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v_cache + tile, ok ? TILE : 0);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      kk[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, lane * 16 + i * 1024, 0, CP));
#pragma unroll
    for (int i = 0; i < NI; ++i)
      vv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, lane * 16 + i * 1024, 0, CP));
  };
  uint32_t acc = 0;
  auto consume = [&](const u32x4* kk, const u32x4* vv) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i) acc ^= fold(kk[i]) ^ fold(vv[i]);
  };

  u32x4 ka[NI], va[NI], kb[NI], vb[NI];
  for (cb = b0; cb < b1; cb += kWave) {
    ce = min(cb + kWave, b1);
    tbl = (cb + lane < ce) ? trow[cb + lane] : -1;
    int j = cb + wave;
    if (j >= ce) break;
    issue(j, ka, va);
    while (true) {
      issue(j + NW, kb, vb);
      consume(ka, va);
      j += NW;
      if (j >= ce) break;
      issue(j + NW, ka, va);
      consume(kb, vb);
      j += NW;
      if (j >= ce) break;
    }
  }
  for (int s = 1; s < kWave; s <<= 1) acc ^= uint32_t(__shfl_xor(int(acc), s));
  if (lane == 0) p.out[int64_t(blockIdx.x) * NW + wave] = acc;
}

// The LDS-staged form: a tile of NI KiB (K and V) per stage and wave; the two
// stages are distinct LDS arrays, so the compiler's wait before reading one
// covers only the loads into that one and the other stays in flight.
constexpr int kLdsTileMax = 4096;

template <int NI, int NW>
__global__ __launch_bounds__(kWave* NW) void gather_probe_lds_kernel(const ProbeParams p) {
  static_assert(NI * 1024 <= kLdsTileMax, "LDS stages hold tiles of at most 4 KiB");
  __shared__ __attribute__((aligned(16))) char st_a[NW][2 * NI * 1024];
  __shared__ __attribute__((aligned(16))) char st_b[NW][2 * NI * 1024];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wi = blockIdx.x / p.num_kv_heads;
  const int kvh = blockIdx.x - wi * p.num_kv_heads;
  const int seq = p.work[2 * wi];
  const int part = p.work[2 * wi + 1];
  const int L = p.context_lens[seq];
  const int nblk = min((L + kBlockTokens - 1) / kBlockTokens, p.table_stride);
  const int b0 = part * p.partition_blocks;
  const int b1 = min(b0 + p.partition_blocks, nblk);
  const int32_t* trow = p.block_tables + int64_t(seq) * p.table_stride;
  const int TILE = NI * 1024;
  const int64_t blk_stride = int64_t(p.num_kv_heads) * TILE;

  int cb = 0, ce = 0, tbl = -1;
  // K then V of block j into stage S: lane l's 16 bytes of load i land at
  // byte 1024 i + 16 l of the stage's K (or V) half, the tile's own layout.
  auto issue = [&](auto stage, int j) __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
    const int blk = __builtin_amdgcn_readlane(tbl, min(j - cb, kWave - 1));
    const bool ok = j < ce && unsigned(blk) < unsigned(p.num_blocks);
    const int64_t tile = int64_t(ok ? blk : 0) * blk_stride + int64_t(kvh) * TILE;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k_cache + tile, ok ? TILE : 0);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v_cache + tile, ok ? TILE : 0);
    char* base = S == 0 ? &st_a[wave][0] : &st_b[wave][0];
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(base + i * 1024), 16,
                                               lane * 16 + i * 1024, 0, 0, kCachePolicyNT);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(base + TILE + i * 1024),
                                               16, lane * 16 + i * 1024, 0, 0, kCachePolicyNT);
  };
  uint32_t acc = 0;
  auto consume = [&](auto stage) __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
    const char* base = S == 0 ? &st_a[wave][0] : &st_b[wave][0];
#pragma unroll
    for (int i = 0; i < 2 * NI; ++i) acc ^= fold(*reinterpret_cast<const u32x4*>(base + i * 1024 + lane * 16));
  };
  using A = std::integral_constant<int, 0>;
  using B = std::integral_constant<int, 1>;

  for (cb = b0; cb < b1; cb += kWave) {
    ce = min(cb + kWave, b1);
    tbl = (cb + lane < ce) ? trow[cb + lane] : -1;
    int j = cb + wave;
    if (j >= ce) break;
    issue(A{}, j);
    while (true) {
      issue(B{}, j + NW);
      consume(A{});
      j += NW;
      if (j >= ce) break;
      issue(A{}, j + NW);
      consume(B{});
      j += NW;
      if (j >= ce) break;
    }
  }
  for (int s = 1; s < kWave; s <<= 1) acc ^= uint32_t(__shfl_xor(int(acc), s));
  if (lane == 0) p.out[int64_t(blockIdx.x) * NW + wave] = acc;
}

using ProbeFn = void (*)(const ProbeParams);

template <int NW>
ProbeFn pick_probe(int ni, int mode) {
  if (mode == PKV_PROBE_LDS) {
    switch (ni) {
      case 2: return gather_probe_lds_kernel<2, NW>;
      case 4: return gather_probe_lds_kernel<4, NW>;
      default: return nullptr;
    }
  }
  const bool cached = mode == PKV_PROBE_CACHED;
  switch (ni) {
    case 2: return cached ? gather_probe_kernel<2, 0, NW> : gather_probe_kernel<2, kCachePolicyNT, NW>;
    case 4: return cached ? gather_probe_kernel<4, 0, NW> : gather_probe_kernel<4, kCachePolicyNT, NW>;
    case 8: return cached ? gather_probe_kernel<8, 0, NW> : gather_probe_kernel<8, kCachePolicyNT, NW>;
    case 16: return cached ? gather_probe_kernel<16, 0, NW> : gather_probe_kernel<16, kCachePolicyNT, NW>;
    default: return nullptr;
  }
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" pkv_status pkv_gather_probe(const pkv_pool* pool, const int32_t* block_tables, int32_t table_stride,
                                       const int32_t* context_lens, int32_t num_seqs, const int32_t* plan,
                                       const pkv_decode_plan_info* info, int32_t mode, int32_t waves,
                                       int32_t lds_pad, uint32_t* out, void* stream) {
  if (!pool || !info) return fail(PKV_E_BAD_ARG, "null pool or plan info");
  const pkv_pool_desc& d = pool->desc;
  if (!pool->k_cache || !pool->v_cache) return fail(PKV_E_BAD_ARG, "pool has no device K/V arrays");
  if (d.block_size != kBlockTokens) return fail(PKV_E_UNSUPPORTED, "block_size 16 only");
  if (mode != PKV_PROBE_REGS && mode != PKV_PROBE_CACHED && mode != PKV_PROBE_LDS)
    return fail(PKV_E_BAD_ARG, "unknown probe mode");
  if (waves != 1 && waves != 2 && waves != 4) return fail(PKV_E_BAD_ARG, "waves must be 1, 2 or 4");
  if (lds_pad < 0 || lds_pad > 65536) return fail(PKV_E_BAD_ARG, "lds_pad must be in [0, 65536]");
  if (info->num_seqs != num_seqs || info->block_size != d.block_size || info->n_work < 0 ||
      info->partition_tokens < kBlockTokens || info->partition_tokens % kBlockTokens != 0)
    return fail(PKV_E_BAD_ARG, "plan info does not match this batch");
  if (info->n_nodes > 0) return fail(PKV_E_UNSUPPORTED, "the probe takes plans without shared-block nodes");
  if (table_stride < 1 || int64_t(info->max_context_len) > int64_t(table_stride) * kBlockTokens)
    return fail(PKV_E_BAD_ARG, "a context is longer than its table can address");
  const int tile = kBlockTokens * d.head_dim * dtype_bytes(d.dtype);
  const int ni = tile / 1024;
  ProbeFn fn = nullptr;
  if (tile % 1024 == 0)
    fn = waves == 1 ? pick_probe<1>(ni, mode) : waves == 2 ? pick_probe<2>(ni, mode) : pick_probe<4>(ni, mode);
  if (!fn) return fail(PKV_E_UNSUPPORTED, "no probe instance for this tile size and mode");
  if (num_seqs == 0 || info->n_work == 0) return PKV_OK;
  if (!block_tables || !context_lens || !plan || !out) return fail(PKV_E_BAD_ARG, "null device pointer");
  if (int64_t(info->n_work) * d.num_kv_heads > INT32_MAX) return fail(PKV_E_BAD_ARG, "batch too large");
  ProbeParams p;
  p.k_cache = static_cast<const char*>(pool->k_cache);
  p.v_cache = static_cast<const char*>(pool->v_cache);
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.work = plan;
  p.out = out;
  p.num_kv_heads = d.num_kv_heads;
  p.table_stride = table_stride;
  p.num_blocks = d.num_blocks;
  p.partition_blocks = info->partition_tokens / kBlockTokens;
  p.tile_bytes = tile;
  const uint32_t grid = uint32_t(int64_t(info->n_work) * d.num_kv_heads);
  hipLaunchKernelGGL(fn, dim3(grid), dim3(kWave * waves), size_t(lds_pad), static_cast<hipStream_t>(stream), p);
  return launch_status("gather probe");
}
