// Chunk pipeline shared by the bf16 attention kernels (gfx950).
//
// A "chunk" is 64 consecutive rows of two [T, D] bf16 matrices (K and V in
// the forward and dQ kernels, Q and dO in the dK/dV kernel) plus up to four
// 64-entry int/float vectors (positions, buckets, lse, D).  Chunks are copied
// global -> LDS with global_load_lds_dwordx4 (lane l's 16 bytes land at
// dst + 16*l whatever the source address), double-buffered, so no VGPRs or
// ds_write instructions are spent on staging.
//
// LDS layout of a matrix: row-major, 16-byte pieces XOR-swizzled inside each
// row: logical piece c of row r sits at physical piece c ^ swz<D>(r).  The LDS
// serves 256 bytes per pass: 16 lanes of a 16-byte row-fragment read, 32 lanes
// of an 8-byte transposed read.
//  * D = 64 (128-byte rows, 8 pieces): row bits 1, 2, 3 flip piece bits 2, 0,
//    1.  A row-fragment read (rows r..r+15, one logical piece) then reaches 16
//    different bank groups, and so does each pass of a transposed read (rows
//    4h..4h+3 or the same + 8, at logical piece pairs): neither conflicts.  (A
//    swizzle over r & 7 alone, which rows r and r + 8 share, cost every
//    row-fragment read four cycles of conflicts.)
//  * D = 128 (256-byte rows, 16 pieces): the swizzle is r & 15 with its four
//    bits reversed; every row starts on the same bank, so the 16 rows of a
//    row-fragment pass need 16 different pieces, and the transposed reads'
//    passes stay conflict-free as well.  (A 3-bit swizzle over r & 7 left
//    four cycles of conflicts on every row-fragment read and two on every
//    transposed one.)
// Either way rows r and r + 16 share the swizzle and rows r and r + 8 do not.
// The swizzle is applied through the DMA source addresses.
// Rows past the end of the sequence are filled with copies of the last real
// row (finite values); the kernels mask them explicitly.
//
// Fragment reads for v_mfma_f32_32x32x16_bf16 (lane l, col = l % 32,
// half = l / 32):
//  * frag_rows: A operand whose rows are chunk rows (row r = 32*sub + col,
//    k = 8 consecutive columns 16*kk + 8*half ..): one ds_read_b128.
//  * frag_trans: A operand whose rows are matrix COLUMNS (column
//    32*mt + col) and whose k items are 8 chunk rows: rows 16t + 4*half + 0..3
//    (items 0..3) and 16t + 8 + 4*half + 0..3 (items 4..7), built from two
//    ds_read_b64_tr_b16.  That row order is exactly the order in which a C
//    tile's registers 8t'..8t'+7 (rows 8*(r/4) + 4*half + r%4) hold their
//    rows, so a C tile converted to bf16 is the matching B operand.
//    ds_read_b64_tr_b16 within each group of 16 lanes returns to lane 4a+b
//    element b of the 8-byte pieces read by lanes a, a+4, a+8, a+12.
#pragma once

#include "scfa_device.hpp"

namespace scfa {

// Piece swizzle of row r for rows of D bf16 values.
template <int D>
__device__ __forceinline__ constexpr int swz(int r) {
  if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 1) | (((r >> 3) & 1) << 1);
  else return ((r & 1) << 3) | ((r & 2) << 1) | ((r & 4) >> 1) | ((r & 8) >> 3);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ lds_void *to_lds(const void *p) {
  return (lds_void *)(p);  // generic -> LDS address space (the pointer is an LDS pointer)
}

// Wait until this wave's outstanding vector-memory operations (including
// global->LDS copies) have completed: s_waitcnt vmcnt(0) (expcnt and lgkmcnt
// fields at their maxima, i.e. not waited for).  Issued through the builtin so
// the compiler's wait-count pass sees it and knows that every earlier load has
// landed; an asm wait would leave loads issued before the chunk loop looking
// outstanding inside it, and the pass would then wait for the loop's own
// loads.
__device__ __forceinline__ void wait_vmem() {
#if defined(__HIP_DEVICE_COMPILE__)  // target builtin: device pass only
  __builtin_amdgcn_s_waitcnt(0x0F70);
#endif
}

// A block's live list (row list: key blocks of a query block; column list:
// query blocks of a key block).  Stored entries are read through a register
// window: lane l holds entry base + l, so entry t costs one v_readlane and the
// chunk loop issues no list loads (a load there would be waited for together
// with the chunk copies in flight).  The window moves forward 64 entries at a
// time; lists are walked in increasing t.
struct LiveList {
  int n;             // live entries
  int first;         // dense-causal column lists: first live query block
  const int32_t *p;  // stored entries (pruned modes), a row of `lim` slots; else nullptr
  int lim;           // slots in the stored row (entries past n are never used)
  int base;          // first entry held in win
  int win;           // this lane's entry p[base + lane] (0 past lim)
};

// The empty asm consumes the loaded value where it is issued, so the wait for
// it happens here (once per 64 entries) and the readlane in the chunk loop has
// no load outstanding; without it the wait lands in the loop and also drains
// the chunk copies in flight.
__device__ __forceinline__ void list_window(LiveList &l, int base) {
  l.base = base;
  const int i = base + (int)(threadIdx.x & 63);
  l.win = i < l.lim ? l.p[i] : 0;
  asm volatile("" : "+v"(l.win));
}

// Two windows loaded together, so their loads share one wait.
__device__ __forceinline__ void list_window2(LiveList &l, LiveList &m, int base) {
  l.base = m.base = base;
  const int i = base + (int)(threadIdx.x & 63);
  l.win = i < l.lim ? l.p[i] : 0;
  m.win = i < m.lim ? m.p[i] : 0;
  asm volatile("" : "+v"(l.win), "+v"(m.win));
}

// Stored entry t (t >= base; uniform across the wave).
__device__ __forceinline__ int list_entry(LiveList &l, int t) {
  if (t - l.base >= 64) list_window(l, t & ~63);
  return __builtin_amdgcn_readlane(l.win, t - l.base);
}

// Global -> LDS copies (lane l's `size` bytes land at dst + size*l, M0 holding
// dst).  They are issued as inline asm, not through the compiler builtin: the
// compiler's wait-count pass cannot tell which LDS bytes a builtin copy
// writes, so it made every LDS read wait for all copies in flight, including
// the next chunk's copy into the other buffer, which serialised the double
// buffer.  Hidden in asm, a copy is waited for only where the kernels say so:
// the vmcnt(0) + barrier at the top of each chunk loop, which every read of
// copied data follows.  (Vector-memory loads complete in order, so the
// compiler's own waits for register loads stay correct with these in the
// count.)  Nothing else in these kernels uses M0; the s_nop is the wait state
// between the M0 write and the copy.
__device__ __forceinline__ void lds_copy16(const void *src, void *dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)to_lds(dst));  // dst is wave-uniform
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory");
}

// The same copies from a wave-uniform base (held in SGPRs) plus a per-lane
// 32-bit byte offset: the address needs no 64-bit vector arithmetic, and
// copies from two matrices at the same rows share one offset register.
// (readfirstlane returns a signed int: each half goes through uint32_t before
// widening, or a low word with bit 31 set would fill the high word with ones.)
__device__ __forceinline__ uint64_t uniform_base(const void *p) {
  const uint64_t b = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}
__device__ __forceinline__ void lds_copy16_at(uint64_t base, uint32_t off, void *dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)to_lds(dst));  // dst is wave-uniform
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(m0)
               : "memory");
}
__device__ __forceinline__ void lds_copy4_at(uint64_t base, uint32_t off, void *dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)to_lds(dst));  // dst is wave-uniform
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(m0)
               : "memory");
}

// The wave's index in its group, known to the compiler as wave-uniform, so the
// LDS destinations of the copies are computed with scalar instructions.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Hardware dispatches work group i to XCD i % 8.  Give each XCD a contiguous
// range of logical ids so the blocks of one head share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int q = n / 8, r = n % 8;
  const int xcd = i % 8, slot = i / 8;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

template <int D>
struct MatChunk {
  uint16_t v[kChunk * D];
};

// Per-lane source offsets (elements, relative to row0) of this wave's DMA
// pieces of a full chunk; a chunk copy is then one 64-bit add per piece.
template <int D, int NW>
struct DmaOffsets {
  static constexpr int CPR = D / 8;
  static constexpr int NINST = kChunk * CPR / 64;  // 16-byte-piece instructions per chunk
  static constexpr int PER_WAVE = (NINST + NW - 1) / NW;
  int off[PER_WAVE];
};

template <int D, int NW>
__device__ __forceinline__ DmaOffsets<D, NW> dma_offsets() {
  using O = DmaOffsets<D, NW>;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  O o;
#pragma unroll
  for (int k = 0; k < O::PER_WAVE; ++k) {
    const int i = k * NW + w;
    const int s = i * 64 + lane;
    const int r = s / O::CPR, p = s % O::CPR;
    o.off[k] = r * D + ((p ^ swz<D>(r)) << 3);
  }
  return o;
}

// Copy rows row0 .. row0+63 of g ([T, D], this head) into an LDS chunk.
// Rows at or past row0 + nvalid repeat row row0 + nvalid - 1 (nvalid >= 1).
// Work is split over the NW waves of the group: 16-byte pieces, 64 per
// instruction.
template <int D, int NW>
__device__ __forceinline__ void dma_matrix(MatChunk<D> &dst, const uint16_t *g, int row0, int nvalid,
                                           const DmaOffsets<D, NW> &o) {
  using O = DmaOffsets<D, NW>;
  const int lane = threadIdx.x & 63, w = wave_id();
  const uint64_t base = uniform_base(g + (size_t)row0 * D);
  if (nvalid == kChunk) {  // wave-uniform: one branch for the whole chunk
#pragma unroll
    for (int k = 0; k < O::PER_WAVE; ++k) {
      const int i = k * NW + w;
      if (O::NINST % NW == 0 || i < O::NINST) {
        lds_copy16_at(base, (uint32_t)o.off[k] * 2u, dst.v + i * 512);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < O::PER_WAVE; ++k) {
      const int i = k * NW + w;
      if (O::NINST % NW == 0 || i < O::NINST) {
        const int s = i * 64 + lane;
        const int r = s / O::CPR, p = s % O::CPR;
        const int rr = r < nvalid ? r : nvalid - 1;
        lds_copy16_at(base, (uint32_t)(rr * D + ((p ^ swz<D>(r)) << 3)) * 2u, dst.v + i * 512);
      }
    }
  }
}

// Row indirection: the source rows this lane copies in each of its DMA
// instructions for one chunk, read from rows[row0 ..] (tail rows repeat the
// last real one).  Loaded one chunk ahead of the copy that uses them;
// dma_matrix_rows clamps them into [0, T) so a bad index cannot leave the
// head's matrix.
template <int D, int NW>
struct DmaRows {
  int row[DmaOffsets<D, NW>::PER_WAVE];
};

template <int D, int NW>
__device__ __forceinline__ void dma_rows_load(DmaRows<D, NW> &dr, const int32_t *rows, int row0, int nvalid) {
  using O = DmaOffsets<D, NW>;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < O::PER_WAVE; ++k) {
    const int i = k * NW + w;
    const int r = (i * 64 + lane) / O::CPR;
    dr.row[k] = rows[row0 + min(r, nvalid - 1)];
  }
}

// dma_matrix through the row indirection: g is the head's matrix base.  The
// byte offset of a row is 32-bit: the host accepts B * H * T * D < 2^31
// elements, so a head's bf16 matrix spans less than 4 GiB.
template <int D, int NW>
__device__ __forceinline__ uint32_t dma_row_offset(const DmaRows<D, NW> &dr, int k, int T) {
  // The piece part depends on the thread only (unsigned, from threadIdx), so it
  // is computed once outside the chunk loop; per chunk: a clamp and a shift-add.
  constexpr unsigned CPR = DmaOffsets<D, NW>::CPR;
  const unsigned s = ((unsigned)k * NW + (threadIdx.x >> 6)) * 64u + (threadIdx.x & 63u);
  const unsigned r = s / CPR, p = s % CPR;
  const unsigned piece = (p ^ (unsigned)swz<D>((int)r)) << 4;
  const int src = min(max(dr.row[k], 0), T - 1);
  return (uint32_t)src * (uint32_t)(D * 2) + piece;
}

template <int D, int NW>
__device__ __forceinline__ void dma_matrix_rows(MatChunk<D> &dst, const uint16_t *g, int T, const DmaRows<D, NW> &dr) {
  using O = DmaOffsets<D, NW>;
  const int w = wave_id();
  const uint64_t base = uniform_base(g);
#pragma unroll
  for (int k = 0; k < O::PER_WAVE; ++k) {
    const int i = k * NW + w;
    if (O::NINST % NW == 0 || i < O::NINST) lds_copy16_at(base, dma_row_offset<D, NW>(dr, k, T), dst.v + i * 512);
  }
}

// Copy 64 consecutive 4-byte values (clamped like dma_matrix) with one wave.
__device__ __forceinline__ void dma_vec(void *dst, const void *g, int row0, int nvalid) {
  const int lane = threadIdx.x & 63;
  const int rr = lane < nvalid ? lane : nvalid - 1;
  lds_copy4_at(uniform_base(static_cast<const uint32_t *>(g) + row0), (uint32_t)rr * 4u, dst);
}

// Lane offset of frag_trans(mt, t = 0): its first read (second = 0, rows
// 4h..4h+3) or its second (second = 1, the same rows + 8).
template <int D>
__device__ __forceinline__ int trans_offset(int mt, int second) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, a = j & 3, mm = j >> 2, g = lane >> 4, h = g >> 1;
  const int r = 4 * h + mm + 8 * second;
  const int c = 4 * mt + 2 * (g & 1) + (a >> 1);
  return r * D + ((c ^ swz<D>(r)) << 3) + 4 * (a & 1);
}

// Per-lane element offsets of the fragment reads inside a MatChunk<D>, computed
// once per kernel so every read in the main loop is base + lane offset +
// compile-time constant (an LDS instruction immediate).
//  rows[kk]: frag_rows(row = col, kk); add 32*sub*D for sub-tile sub.
//  trans[mt]: first read of frag_trans(mt, t = 0); add 16*t*D for k-step t
//             (rows r and r + 16 share the swizzle).
//  trans2[mt]: its second read (row r + 8, whose swizzle differs).
template <int D>
struct LaneOffsets {
  int rows[D / 16];
  int trans[D / 32];
  int trans2[D / 32];
};

template <int D>
__device__ __forceinline__ LaneOffsets<D> lane_offsets() {
  const int lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  LaneOffsets<D> o;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) o.rows[kk] = col * D + (((2 * kk + half) ^ swz<D>(col)) << 3);
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) {
    o.trans[mt] = trans_offset<D>(mt, 0);
    o.trans2[mt] = trans_offset<D>(mt, 1);
  }
  return o;
}

template <int D>
__device__ __forceinline__ bf16x8 frag_rows(const MatChunk<D> &m, const LaneOffsets<D> &o, int sub, int kk) {
  return as_bf16x8(*reinterpret_cast<const uint4 *>(m.v + o.rows[kk] + 32 * sub * D));
}

// A operand over matrix columns 32*mt + (l % 32) and chunk rows of k-step t.
template <int D>
__device__ __forceinline__ bf16x8 frag_trans(const MatChunk<D> &m, const LaneOffsets<D> &o, int mt, int t) {
  const uint16_t *p0 = m.v + o.trans[mt] + 16 * t * D;
  const uint16_t *p1 = m.v + o.trans2[mt] + 16 * t * D;
#if defined(__HIP_DEVICE_COMPILE__)  // target builtin: device pass only
  const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)to_lds(p0));
  const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)to_lds(p1));
#else
  const i16x4 x0 = {}, x1 = {};
#endif
  const uint2 lo = __builtin_bit_cast(uint2, x0), hi = __builtin_bit_cast(uint2, x1);
  return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// frag_trans with the lane offsets given directly (trans_offset<D>(mt, 0 / 1)).
template <int D>
__device__ __forceinline__ bf16x8 frag_trans_at(const MatChunk<D> &m, int off, int off2, int t) {
  const uint16_t *p0 = m.v + off + 16 * t * D;
  const uint16_t *p1 = m.v + off2 + 16 * t * D;
#if defined(__HIP_DEVICE_COMPILE__)  // target builtin: device pass only
  const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)to_lds(p0));
  const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)to_lds(p1));
#else
  const i16x4 x0 = {}, x1 = {};
#endif
  const uint2 lo = __builtin_bit_cast(uint2, x0), hi = __builtin_bit_cast(uint2, x1);
  return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Sum of eight bf16 values packed in a uint4, accumulated into acc (fp32)
// with v_dot2 against (1, 1).
__device__ __forceinline__ float add_bf16x8(uint4 u, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.x), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.y), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.z), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.w), one, acc, false);
  return acc;
}

__device__ __forceinline__ uint4 c_regs_to_u4(const f32x16 &c, int t) {
  uint4 u;
  u.x = pack_bf16x2(c[8 * t + 0], c[8 * t + 1]);
  u.y = pack_bf16x2(c[8 * t + 2], c[8 * t + 3]);
  u.z = pack_bf16x2(c[8 * t + 4], c[8 * t + 5]);
  u.w = pack_bf16x2(c[8 * t + 6], c[8 * t + 7]);
  return u;
}

// Element mask over a pair of C tiles whose rows are chunk rows r0 + 32*sub +
// 8g + 4*half + e.  The lane's column is a query (my_idx is a query position,
// rows are keys): admissible iff row_idx <= my_idx.  Hash mode also needs
// equal bucket ids; with TAIL, rows at or past nvalid (copies of a real row)
// are inadmissible.  Inadmissible entries are replaced by `fill`.
// Branch-free (compare + select).
template <int MODE, bool TAIL>
__device__ __forceinline__ void mask_rows(f32x16 (&s)[2], const int *sidx, const int *shash, int r0, int nvalid,
                                          int my_idx, int my_hash, int half, float fill) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int rr = 32 * sub + 8 * g + 4 * half;
      int iv[4], hv[4] = {0, 0, 0, 0};
      if (MODE == kDense) {
#pragma unroll
        for (int e = 0; e < 4; ++e) iv[e] = r0 + rr + e;
      } else {
        const int4 ki = *reinterpret_cast<const int4 *>(sidx + rr);
        iv[0] = ki.x, iv[1] = ki.y, iv[2] = ki.z, iv[3] = ki.w;
        if (MODE == kHash) {
          const int4 kh = *reinterpret_cast<const int4 *>(shash + rr);
          hv[0] = kh.x, hv[1] = kh.y, hv[2] = kh.z, hv[3] = kh.w;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bool ok = iv[e] <= my_idx;
        if (MODE == kHash) ok = ok & (hv[e] == my_hash);
        if (TAIL) ok = ok & (rr + e < nvalid);
        s[sub][4 * g + e] = ok ? s[sub][4 * g + e] : fill;
      }
    }
}

// mask_rows for one C tile whose rows are chunk rows sub0 + 8g + 4*half + e
// (sub0 = 0 or 32) and whose lane column is a query: admissible iff the row's
// key position <= my_idx (dense mode: the position is chunk_r0 + chunk row),
// and equal buckets in hash mode; with TAIL, rows at or past nvalid are
// inadmissible.  Inadmissible entries become `fill`.
template <int MODE, bool TAIL>
__device__ __forceinline__ void mask_tile_q(f32x16 &s, const int *sidx, const int *shash, int sub0, int chunk_r0,
                                            int nvalid, int my_idx, int my_hash, int half, float fill) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int rr = sub0 + 8 * g + 4 * half;
    int iv[4], hv[4] = {0, 0, 0, 0};
    if (MODE == kDense) {
#pragma unroll
      for (int e = 0; e < 4; ++e) iv[e] = chunk_r0 + rr + e;
    } else {
      const int4 ki = *reinterpret_cast<const int4 *>(sidx + rr);
      iv[0] = ki.x, iv[1] = ki.y, iv[2] = ki.z, iv[3] = ki.w;
      if (MODE == kHash) {
        const int4 kh = *reinterpret_cast<const int4 *>(shash + rr);
        hv[0] = kh.x, hv[1] = kh.y, hv[2] = kh.z, hv[3] = kh.w;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bool ok = iv[e] <= my_idx;
      if (MODE == kHash) ok = ok & (hv[e] == my_hash);
      if (TAIL) ok = ok & (rr + e < nvalid);
      s[4 * g + e] = ok ? s[4 * g + e] : fill;
    }
  }
}

// mask_rows for one C tile whose rows are chunk rows sub0 + 8g + 4*half + e
// (sub0 = 0 or 32); the lane's column is a key and rows are queries:
// admissible iff my_idx <= row position (dense mode: the position is
// chunk_r0 + chunk row), and equal buckets in hash mode; with TAIL, rows at
// or past nvalid are inadmissible.  Inadmissible entries become `fill`.
template <int MODE, bool TAIL>
__device__ __forceinline__ void mask_half(f32x16 &s, const int *sidx, const int *shash, int sub0, int chunk_r0,
                                          int nvalid, int my_idx, int my_hash, int half, float fill) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int rr = sub0 + 8 * g + 4 * half;
    int iv[4], hv[4] = {0, 0, 0, 0};
    if (MODE == kDense) {
#pragma unroll
      for (int e = 0; e < 4; ++e) iv[e] = chunk_r0 + rr + e;
    } else {
      const int4 ki = *reinterpret_cast<const int4 *>(sidx + rr);
      iv[0] = ki.x, iv[1] = ki.y, iv[2] = ki.z, iv[3] = ki.w;
      if (MODE == kHash) {
        const int4 kh = *reinterpret_cast<const int4 *>(shash + rr);
        hv[0] = kh.x, hv[1] = kh.y, hv[2] = kh.z, hv[3] = kh.w;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bool ok = my_idx <= iv[e];
      if (MODE == kHash) ok = ok & (hv[e] == my_hash);
      if (TAIL) ok = ok & (rr + e < nvalid);
      s[4 * g + e] = ok ? s[4 * g + e] : fill;
    }
  }
}

}  // namespace scfa
