// Device-side helpers shared by the gfx950 kernels: bf16 vector types, the
// 32x32x16 bf16 matrix-core instruction, wave-level exchange, float helpers.
//
// Operand layout facts of v_mfma_f32_32x32x16_bf16 on a 64-lane wave (lane l,
// col = l % 32, half = l / 32):
//   A (32 x 16): lane holds row `col`, 8 consecutive k of half `half`.
//   B (16 x 32): lane holds column `col`, the same 8 k of half `half`.
//   C (32 x 32): lane holds column `col`; register r holds row
//                8*(r/4) + 4*half + (r%4).
// Any bijection between (half, item) and the contraction index works as long
// as A and B use the same one; the kernels exploit this to feed a C tile back
// in as a B operand without moving data between lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace scfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr f32x16 kZero16 = {};
constexpr int kIdxTailQ = INT32_MIN;  // position of a query row past Tq: no key precedes it
constexpr int kIdxTailK = INT32_MAX;  // position of a key row past Tk: follows every query

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void st16(void *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }

// Value of lane l ^ 32 combined with the own value (max or sum) for every lane.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Round-to-nearest-even float -> bf16 bit patterns, two at a time (v_cvt_pk_bf16_f32).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

constexpr int kChunk = 64;  // rows of a streamed chunk

}  // namespace scfa
