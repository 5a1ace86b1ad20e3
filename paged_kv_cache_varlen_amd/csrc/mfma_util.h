// Device helpers shared by the attention kernels (attend.hip, mla.hip):
// vector types, the two bf16 MFMA shapes they use, and the column maximum of
// an MFMA output tile.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// 16x16x32 bf16 MFMA: lane (r, g) holds A[r][8g..8g+7] and B[8g..8g+7][r];
// the result lane holds C[4g..4g+3][r].
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x16 bf16 MFMA: lane (r, g) holds A[r][4g..4g+3] and B[4g..4g+3][r].
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
      __builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Maximum over the four lanes r, r + 16, r + 32, r + 48, which hold the
// rows of MFMA column r: two VALU lane swaps (no LDS round trip).
__device__ __forceinline__ float column_max(float x) {
  const uint32_t xb = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(xb, xb, false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t yb = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane16_swap(yb, yb, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

}  // namespace
}  // namespace pa
