// Matrix-core helpers shared by the decode and prefill kernels (gfx950).
//
// Operand layouts of the 16x16 products used here (lane l = 16 g + n):
//  * v_mfma_f32_16x16x32_{f16,bf16}: lane l holds A[row n][k = 8 g .. 8 g + 7]
//    and B[k = 8 g .. 8 g + 7][column n] (16 bytes each);
//  * v_mfma_f32_16x16x16_{f16,bf16}: the same with k = 4 g .. 4 g + 3 (8 bytes);
//  * both leave lane l with C[rows 4 g .. 4 g + 3][column n] (four fp32).
// The accumulator layout is therefore the B-operand layout of a following
// 16x16x16 product (and, two blocks side by side, of a 16x16x32 one).
#pragma once

#include "device_common.h"

namespace pkv {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegBig = -3.0e38f;  // finite "nothing seen yet" running maximum

// C += A B with 16x16x32 operands of 16-bit elements (fp32 accumulation).
template <int DT>
__device__ __forceinline__ f4 mfma_k32(const u32x4& a, const u32x4& b, const f4& c) {
  if constexpr (DT == PKV_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c,
                                                   0, 0, 0);
}

// C += A B with 16x16x16 operands of 16-bit elements (fp32 accumulation).
template <int DT>
__device__ __forceinline__ f4 mfma_k16(const u32x2& a, const u32x2& b, const f4& c) {
  if constexpr (DT == PKV_F16)
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4, a), __builtin_bit_cast(h4, b), c, 0, 0,
                                                 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a), __builtin_bit_cast(s4, b), c,
                                                     0, 0, 0);
}

// Maximum over the four lanes n, n + 16, n + 32, n + 48 (one accumulator
// column), with gfx950's lane swaps instead of LDS permutes: a swap of a
// register with itself leaves, in the two results, each lane's own value and
// its partner's (16 lanes away for permlane16, 32 for permlane32).  The two
// results are copied into scalars before they are reinterpreted as floats:
// this compiler lowers a bit_cast of an element of the returned vector as a
// read of element 0, so the second result would silently become the first
// and the maximum would cover only lanes 0-15 (see device_common.h).
__device__ __forceinline__ float max_over_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const uint32_t a0 = a[0], a1 = a[1];
  x = fmaxf(__uint_as_float(a0), __uint_as_float(a1));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const uint32_t b0 = b[0], b1 = b[1];
  return fmaxf(__uint_as_float(b0), __uint_as_float(b1));
}

}  // namespace pkv
