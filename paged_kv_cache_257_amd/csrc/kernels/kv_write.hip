// write_kv, read_kv and copy_blocks: the device half of appending tokens
// to a paged KV cache and of reading them back.
//
// write_kv stores each new token's K and V rows at the slot the allocator
// handed out ("04 — Hacia PagedAttention", La idea de PagedAttention, step 3:
// a token goes into the last block, or a newly taken one).  copy_blocks is
// the copy of copy-on-write ("PagedAttention e continuous batching",
// 01 · Conceito, paragraph 6): the diverging sequence gets its own copy of a
// shared block before it writes.
//
// Both are plain byte moves: each thread moves one 16-byte chunk with a
// 128-bit load and store; the threads of a wave cover consecutive chunks of
// one (token, head) row or one block, so loads and stores are coalesced.
#include <algorithm>

#include "../host/hybrid_internal.h"
#include "device_common.h"

namespace pkv {
namespace {

__global__ __launch_bounds__(256) void write_kv_kernel(const char* __restrict__ k_new,
                                                       const char* __restrict__ v_new,
                                                       const int64_t* __restrict__ slots,
                                                       char* __restrict__ k_cache,
                                                       char* __restrict__ v_cache,
                                                       int64_t n_chunks, int32_t heads,
                                                       int32_t chunks_per_row, int64_t num_slots) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= n_chunks) return;
  const int64_t per_token = int64_t(heads) * chunks_per_row;
  const int64_t t = idx / per_token;
  const int64_t rem = idx - t * per_token;  // = h * chunks_per_row + c
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t h = rem / chunks_per_row;
  const int64_t c = rem - h * chunks_per_row;
  const int64_t blk = slot / kBlockTokens;
  const int64_t row = slot - blk * kBlockTokens;
  const int64_t row_bytes = int64_t(chunks_per_row) * 16;
  const int64_t src = idx * 16;  // token-major source: ((t*H + h)*row + c)
  const int64_t dst = ((blk * heads + h) * kBlockTokens + row) * row_bytes + c * 16;
  *reinterpret_cast<u32x4*>(k_cache + dst) = *reinterpret_cast<const u32x4*>(k_new + src);
  *reinterpret_cast<u32x4*>(v_cache + dst) = *reinterpret_cast<const u32x4*>(v_new + src);
}

// The inverse of write_kv: row t of the dense output is the pool row at
// slot t (zeros for a slot outside the pool).  Same thread-to-chunk map.
__global__ __launch_bounds__(256) void read_kv_kernel(const int64_t* __restrict__ slots,
                                                      const char* __restrict__ k_cache,
                                                      const char* __restrict__ v_cache,
                                                      char* __restrict__ k_out,
                                                      char* __restrict__ v_out, int64_t n_chunks,
                                                      int32_t heads, int32_t chunks_per_row,
                                                      int64_t num_slots) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= n_chunks) return;
  const int64_t per_token = int64_t(heads) * chunks_per_row;
  const int64_t t = idx / per_token;
  const int64_t rem = idx - t * per_token;
  const int64_t slot = slots[t];
  const int64_t dst = idx * 16;
  if (slot < 0 || slot >= num_slots) {
    *reinterpret_cast<u32x4*>(k_out + dst) = u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(v_out + dst) = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const int64_t h = rem / chunks_per_row;
  const int64_t c = rem - h * chunks_per_row;
  const int64_t blk = slot / kBlockTokens;
  const int64_t row = slot - blk * kBlockTokens;
  const int64_t src = ((blk * heads + h) * kBlockTokens + row) * (int64_t(chunks_per_row) * 16) + c * 16;
  *reinterpret_cast<u32x4*>(k_out + dst) = *reinterpret_cast<const u32x4*>(k_cache + src);
  *reinterpret_cast<u32x4*>(v_out + dst) = *reinterpret_cast<const u32x4*>(v_cache + src);
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(const int32_t* __restrict__ pairs,
                                                          char* __restrict__ k_cache,
                                                          char* __restrict__ v_cache,
                                                          int64_t block_bytes, int32_t groups_per_pair,
                                                          int32_t num_blocks) {
  const int32_t pair = blockIdx.x / groups_per_pair;
  const int32_t g = blockIdx.x - pair * groups_per_pair;
  const int32_t src = pairs[2 * pair];
  const int32_t dst = pairs[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const char* ks = k_cache + int64_t(src) * block_bytes;
  const char* vs = v_cache + int64_t(src) * block_bytes;
  char* kd = k_cache + int64_t(dst) * block_bytes;
  char* vd = v_cache + int64_t(dst) * block_bytes;
  for (int64_t off = (int64_t(g) * 256 + threadIdx.x) * 16; off < block_bytes;
       off += int64_t(groups_per_pair) * 256 * 16) {
    *reinterpret_cast<u32x4*>(kd + off) = *reinterpret_cast<const u32x4*>(ks + off);
    *reinterpret_cast<u32x4*>(vd + off) = *reinterpret_cast<const u32x4*>(vs + off);
  }
}

// Whole-slot copies of the hybrid manager's per-sequence state (a forked
// sequence starts from its parent's state).  Same shape as copy_blocks.
__global__ __launch_bounds__(256) void copy_states_kernel(const int32_t* __restrict__ pairs,
                                                          char* __restrict__ base, int64_t slot_bytes,
                                                          int32_t groups_per_pair, int32_t num_slots) {
  const int32_t pair = blockIdx.x / groups_per_pair;
  const int32_t g = blockIdx.x - pair * groups_per_pair;
  const int32_t src = pairs[2 * pair];
  const int32_t dst = pairs[2 * pair + 1];
  if (src < 0 || src >= num_slots || dst < 0 || dst >= num_slots || src == dst) return;
  const char* s = base + int64_t(src) * slot_bytes;
  char* d = base + int64_t(dst) * slot_bytes;
  for (int64_t off = (int64_t(g) * 256 + threadIdx.x) * 16; off < slot_bytes;
       off += int64_t(groups_per_pair) * 256 * 16)
    *reinterpret_cast<u32x4*>(d + off) = *reinterpret_cast<const u32x4*>(s + off);
}

pkv_status check_device_pool(const pkv_pool* p) {
  if (!p) return fail(PKV_E_BAD_ARG, "null pool");
  if (!p->k_cache || !p->v_cache) return fail(PKV_E_BAD_ARG, "pool has no device K/V arrays");
  if (p->desc.block_size != kBlockTokens)
    return fail(PKV_E_UNSUPPORTED, "device kernels take block_size 16 only");
  const int64_t row = int64_t(p->desc.head_dim) * dtype_bytes(p->desc.dtype);
  if (row % 16 != 0) return fail(PKV_E_UNSUPPORTED, "head_dim * element size must be a multiple of 16 bytes");
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" pkv_status pkv_write_kv(const pkv_pool* pool, const void* k_new, const void* v_new,
                                   const int64_t* slot_mapping, int32_t n_tokens, void* stream) {
  if (pkv_status st = check_device_pool(pool)) return st;
  if (n_tokens < 0) return fail(PKV_E_BAD_ARG, "negative n_tokens");
  if (n_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping) return fail(PKV_E_BAD_ARG, "null k_new, v_new or slot_mapping");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
    return fail(PKV_E_BAD_ARG, "k_new and v_new must be 16-byte aligned");
  const pkv_pool_desc& d = pool->desc;
  const int32_t cpr = int32_t(int64_t(d.head_dim) * dtype_bytes(d.dtype) / 16);
  const int64_t n_chunks = int64_t(n_tokens) * d.num_kv_heads * cpr;
  const int64_t grid = (n_chunks + 255) / 256;
  if (grid > INT32_MAX) return fail(PKV_E_BAD_ARG, "write too large for one launch");
  hipLaunchKernelGGL(write_kv_kernel, dim3(uint32_t(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(k_new),
                     static_cast<const char*>(v_new), slot_mapping,
                     static_cast<char*>(pool->k_cache), static_cast<char*>(pool->v_cache), n_chunks,
                     d.num_kv_heads, cpr, int64_t(d.num_blocks) * kBlockTokens);
  return launch_status("write_kv launch");
}

extern "C" pkv_status pkv_read_kv(const pkv_pool* pool, const int64_t* slot_mapping,
                                  int32_t n_tokens, void* k_out, void* v_out, void* stream) {
  if (pkv_status st = check_device_pool(pool)) return st;
  if (n_tokens < 0) return fail(PKV_E_BAD_ARG, "negative n_tokens");
  if (n_tokens == 0) return PKV_OK;
  if (!k_out || !v_out || !slot_mapping) return fail(PKV_E_BAD_ARG, "null k_out, v_out or slot_mapping");
  if ((reinterpret_cast<uintptr_t>(k_out) | reinterpret_cast<uintptr_t>(v_out)) & 15)
    return fail(PKV_E_BAD_ARG, "k_out and v_out must be 16-byte aligned");
  const pkv_pool_desc& d = pool->desc;
  const int32_t cpr = int32_t(int64_t(d.head_dim) * dtype_bytes(d.dtype) / 16);
  const int64_t n_chunks = int64_t(n_tokens) * d.num_kv_heads * cpr;
  const int64_t grid = (n_chunks + 255) / 256;
  if (grid > INT32_MAX) return fail(PKV_E_BAD_ARG, "read too large for one launch");
  hipLaunchKernelGGL(read_kv_kernel, dim3(uint32_t(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), slot_mapping,
                     static_cast<const char*>(pool->k_cache), static_cast<const char*>(pool->v_cache),
                     static_cast<char*>(k_out), static_cast<char*>(v_out), n_chunks, d.num_kv_heads,
                     cpr, int64_t(d.num_blocks) * kBlockTokens);
  return launch_status("read_kv launch");
}

extern "C" pkv_status pkv_copy_blocks(const pkv_pool* pool, const int32_t* pairs, int32_t n_pairs,
                                      void* stream) {
  if (pkv_status st = check_device_pool(pool)) return st;
  if (n_pairs < 0) return fail(PKV_E_BAD_ARG, "negative n_pairs");
  if (n_pairs == 0) return PKV_OK;
  if (!pairs) return fail(PKV_E_BAD_ARG, "null pairs");
  const pkv_pool_desc& d = pool->desc;
  const int64_t block_bytes =
      int64_t(d.num_kv_heads) * kBlockTokens * d.head_dim * dtype_bytes(d.dtype);
  const int64_t chunks = block_bytes / 16;
  const int32_t groups = int32_t(std::min<int64_t>((chunks + 255) / 256, 64));
  const int64_t grid = int64_t(n_pairs) * groups;
  if (grid > INT32_MAX) return fail(PKV_E_BAD_ARG, "too many pairs for one launch");
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(uint32_t(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), pairs, static_cast<char*>(pool->k_cache),
                     static_cast<char*>(pool->v_cache), block_bytes, groups, d.num_blocks);
  return launch_status("copy_blocks launch");
}

extern "C" pkv_status pkv_hybrid_copy_states(pkv_hybrid* h, const int32_t* pairs, int32_t n,
                                             void* stream) {
  if (!h) return fail(PKV_E_BAD_ARG, "null manager");
  if (!h->state_base) return fail(PKV_E_BAD_ARG, "the manager has no device state memory");
  if (n < 0) return fail(PKV_E_BAD_ARG, "negative n");
  if (n == 0) return PKV_OK;
  if (!pairs) return fail(PKV_E_BAD_ARG, "null pairs");
  // enough workgroups per pair to fill the chip for a few pairs, each
  // moving at least 64 KiB
  const int64_t per_group = int64_t(256) * 16 * 16;
  const int32_t gpp = int32_t(std::min<int64_t>(1024, (h->slot_bytes + per_group - 1) / per_group));
  const int64_t grid = int64_t(n) * gpp;
  if (grid > INT32_MAX) return fail(PKV_E_BAD_ARG, "too many pairs");
  hipLaunchKernelGGL(copy_states_kernel, dim3(uint32_t(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), pairs, static_cast<char*>(h->state_base),
                     h->slot_bytes, gpp, h->num_slots);
  return launch_status("copy_states launch");
}
