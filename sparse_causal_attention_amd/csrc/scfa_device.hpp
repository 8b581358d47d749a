// Device-side helpers shared by the gfx950 kernels: bf16 vector types, the
// 32x32x16 bf16 matrix-core instruction, LDS staging of 64-row chunks
// (row-major and transposed), wave-level exchange, and float helpers.
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
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Eight consecutive C-tile registers (8t .. 8t+7) as a bf16 B operand.
__device__ __forceinline__ bf16x8 c_regs_to_bf16x8(const f32x16 &c, int t) {
  uint4 u;
  u.x = pack_bf16x2(c[8 * t + 0], c[8 * t + 1]);
  u.y = pack_bf16x2(c[8 * t + 2], c[8 * t + 3]);
  u.z = pack_bf16x2(c[8 * t + 4], c[8 * t + 5]);
  u.w = pack_bf16x2(c[8 * t + 6], c[8 * t + 7]);
  return as_bf16x8(u);
}

// ---------------------------------------------------------------------------
// LDS staging of a 64-row chunk of a [T, D] bf16 matrix.
//
// Row-major copy: row r at sRow + r*(D+8) elements (16-byte padding per row
// keeps the 16-byte reads of 8 consecutive rows on distinct banks).
//
// Transposed copy: element (r, c) at sT + c*(64+8) + pos(r) where pos permutes
// rows inside each group of 16 so that a lane's 8 contraction items of an
// A operand are contiguous.  Row offset p = 8a + 4b + e (a, b in {0,1},
// e in 0..3) is stored at slot 8b + 4a + e: lane half h, item i of a 16-row
// k-step then reads slot 8h + i, which holds row 8*(i/4) + 4h + (i%4) -- the
// same rows a C tile's registers 8t..8t+7 hold in lane half h.
// ---------------------------------------------------------------------------
constexpr int kChunk = 64;
constexpr int kTPad = kChunk + 8;  // row stride (elements) of a transposed tile

__device__ __forceinline__ int tslot(int r) {
  const int p = r & 15;
  return (r & ~15) + 8 * ((p >> 2) & 1) + 4 * (p >> 3) + (p & 3);
}

template <int D, int NT>
__device__ __forceinline__ void stage_rows(uint16_t *sRow, const uint16_t *g, int row0, int nrows_valid) {
  constexpr int CPR = D / 8;  // 16-byte pieces per row
  for (int i = threadIdx.x; i < kChunk * CPR; i += NT) {
    const int r = i / CPR, c = i % CPR;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (r < nrows_valid) val = ld16(g + (size_t)(row0 + r) * D + c * 8);
    st16(sRow + r * (D + 8) + c * 8, val);
  }
}

template <int D, int NT>
__device__ __forceinline__ void stage_transposed(uint16_t *sT, const uint16_t *g, int row0, int nrows_valid) {
  constexpr int CPR = D / 8;
  // One work item: 4 consecutive rows (4u..4u+3, same slot group) x 8 columns.
  for (int i = threadIdx.x; i < (kChunk / 4) * CPR; i += NT) {
    const int u = i / CPR, c = i % CPR;
    uint4 rows[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * u + e;
      rows[e] = make_uint4(0, 0, 0, 0);
      if (r < nrows_valid) rows[e] = ld16(g + (size_t)(row0 + r) * D + c * 8);
    }
    const int slot = tslot(4 * u);
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const uint32_t w0 = (&rows[0].x)[dd >> 1], w1 = (&rows[1].x)[dd >> 1];
      const uint32_t w2 = (&rows[2].x)[dd >> 1], w3 = (&rows[3].x)[dd >> 1];
      const int sh = (dd & 1) * 16;
      const uint32_t lo = ((w0 >> sh) & 0xffffu) | (((w1 >> sh) & 0xffffu) << 16);
      const uint32_t hi = ((w2 >> sh) & 0xffffu) | (((w3 >> sh) & 0xffffu) << 16);
      *reinterpret_cast<uint2 *>(sT + (c * 8 + dd) * kTPad + slot) = make_uint2(lo, hi);
    }
  }
}

// A operand (rows `row0 + col`, k-step kk) from a row-major staged chunk.
template <int D>
__device__ __forceinline__ bf16x8 lds_a_rows(const uint16_t *sRow, int row, int kk, int half) {
  return as_bf16x8(*reinterpret_cast<const uint4 *>(sRow + row * (D + 8) + 16 * kk + 8 * half));
}

// A operand (row `trow` of the transposed tile, 16-row k-step starting at
// chunk row k0) from a transposed staged chunk.
__device__ __forceinline__ bf16x8 lds_a_trans(const uint16_t *sT, int trow, int k0, int half) {
  return as_bf16x8(*reinterpret_cast<const uint4 *>(sT + trow * kTPad + k0 + 8 * half));
}

}  // namespace scfa
