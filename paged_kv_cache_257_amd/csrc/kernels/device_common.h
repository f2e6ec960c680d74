// Device helpers shared by the libpkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../host/pool_internal.h"

namespace pkv {

constexpr int kWave = 64;
constexpr int kBlockTokens = 16;  // the only block size the kernels take

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int DT>
struct ElemBytes {
  static constexpr int value = (DT == PKV_F32) ? 4 : 2;
};

// Launch-error check for entry points.
inline pkv_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return PKV_OK;
}

__device__ __forceinline__ float bits_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Buffer resource over `bytes` bytes at `base` (raw buffer, no stride): an
// access at an offset >= bytes returns zeros and touches no memory.
constexpr int kBufferFormat = 0x00020000;  // dword3 of a raw gfx9 buffer resource
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferFormat);
}

// 16-byte load of data read once (K/V tiles), with the nontemporal bit set
// ("nt"): it keeps the stream from displacing reusable lines and raises the
// achieved rate of the decode's scattered 4 KiB tile reads on MI355X from
// 5.3-5.7 TB/s (cached loads) to 6.1-6.6 TB/s (pkv_gather_probe).
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ u32x4 load_stream(__amdgpu_buffer_rsrc_t r, int offset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, kCachePolicyNT));
}

// DPP lane move within a row of 16 lanes (all lanes read a valid source for
// the controls used here, so bound_ctrl and the masks do not matter).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return bits_f(uint32_t(__builtin_amdgcn_update_dpp(0, int(f_bits(x)), CTRL, 0xF, 0xF, false)));
}

constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;
constexpr int kRowHalfMirror = 0x141;
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]

// Sum over the N consecutive lanes (N in {8,16,32,64}, aligned) that hold one
// token row; every one of those lanes gets the total.
template <int N>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(N == 8 || N == 16 || N == 32 || N == 64, "row width");
  if constexpr (N == 8) {
    x += dpp<kRowHalfMirror>(x);  // lane i + lane 7-i of each 8
    x += dpp<kQuadSwap2>(x);
    x += dpp<kQuadSwap1>(x);
  } else {
    x += dpp<kRowRor8>(x);  // rotations within 16 lanes: an all-reduce
    x += dpp<kRowRor4>(x);
    x += dpp<kRowRor2>(x);
    x += dpp<kRowRor1>(x);
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    if constexpr (N == 64) x += __shfl_xor(x, 32);
  }
  return x;
}

// Dot product of one 16-byte chunk of q with one of k, accumulated in fp32.
// fp16/bf16 use the two-way dot instructions: products of 16-bit values are
// exact in fp32, the sums are fp32.
template <int DT>
__device__ __forceinline__ float dot16(const u32x4& q, const u32x4& k, float acc);

template <>
__device__ __forceinline__ float dot16<PKV_F32>(const u32x4& q, const u32x4& k, float acc) {
  acc = __builtin_fmaf(bits_f(q.x), bits_f(k.x), acc);
  acc = __builtin_fmaf(bits_f(q.y), bits_f(k.y), acc);
  acc = __builtin_fmaf(bits_f(q.z), bits_f(k.z), acc);
  acc = __builtin_fmaf(bits_f(q.w), bits_f(k.w), acc);
  return acc;
}

// Vector elements are copied into scalars before __builtin_bit_cast: this
// compiler mis-lowers a bit_cast whose operand is an element of an
// ext_vector_type (`q.y`), reading element .x instead.
template <>
__device__ __forceinline__ float dot16<PKV_F16>(const u32x4& q, const u32x4& k, float acc) {
  const uint32_t qa[4] = {q.x, q.y, q.z, q.w};
  const uint32_t ka[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, qa[i]), __builtin_bit_cast(f16x2, ka[i]),
                                 acc, false);
  return acc;
}

template <>
__device__ __forceinline__ float dot16<PKV_BF16>(const u32x4& q, const u32x4& k, float acc) {
  const uint32_t qa[4] = {q.x, q.y, q.z, q.w};
  const uint32_t ka[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qa[i]),
                                          __builtin_bit_cast(bf16x2, ka[i]), acc, false);
  return acc;
}

// The 16/e values of a 16-byte chunk as fp32 (exact conversions).
template <int DT>
__device__ __forceinline__ void to_f32(const u32x4& v, float* f);

template <>
__device__ __forceinline__ void to_f32<PKV_F32>(const u32x4& v, float* f) {
  f[0] = bits_f(v.x); f[1] = bits_f(v.y); f[2] = bits_f(v.z); f[3] = bits_f(v.w);
}

template <>
__device__ __forceinline__ void to_f32<PKV_F16>(const u32x4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f16x2 h = __builtin_bit_cast(f16x2, w[i]);
    f[2 * i] = float(h.x);
    f[2 * i + 1] = float(h.y);
  }
}

template <>
__device__ __forceinline__ void to_f32<PKV_BF16>(const u32x4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bits_f(w[i] << 16);
    f[2 * i + 1] = bits_f(w[i] & 0xFFFF0000u);
  }
}

}  // namespace pkv
