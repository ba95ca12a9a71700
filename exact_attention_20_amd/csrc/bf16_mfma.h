// bf16 matrix-core building blocks shared by the prefill kernels (forward
// and backward): the 32x32x16 bf16 MFMA, the row order that makes an S^T
// accumulator directly usable as a later MFMA's operand, half-wavefront
// reductions and gfx950's transposing LDS read.
#pragma once

#include "hip_common.h"

namespace fa {

// MFMA row r of the S^T tile reads key kperm(r): with it, accumulator
// register i of lane l holds key 16*(i/8) + 8*(l/32) + (i%8).
__device__ __forceinline__ int kperm(int r) {
  const int a = r >> 3, hh = (r >> 2) & 1, c = r & 3;
  return 16 * (a >> 1) + 8 * hh + 4 * (a & 1) + c;
}

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// The same with a zero accumulator (an inline constant: nothing to clear).
__device__ __forceinline__ f32x16_t mfma32_first(bf16x8_t a, bf16x8_t b) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, f32x16_t{}, 0, 0, 0);
}

// x combined with the value of lane ^ 32 (both halves get the result).
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(4))) const int32_t const_i32;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): within each group of 16
// lanes, lane i receives element (i & 3) of the 8-byte chunks addressed by
// lanes 4j + (i >> 2), j = 0..3.
__device__ __forceinline__ uint2 lds_read_tr16(const char* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

}  // namespace fa
