// LSH bucketing and the stable (bucket, original position) reordering that
// feeds Hash-sparse attention (deep-paper.org summary of arXiv 2306.01160:
// "why dynamic sparsity breaks it" -- LSH groups similar tokens into buckets
// as in Reformer, and tokens reordered by hash keep their original positions
// for the causal mask; "2. Hash-Sparse" -- bucket ids per query and key).
//
// Bucket function (random-rotation LSH): p = x . R_h accumulated in float64
// in increasing coordinate order, bucket = first index of max [p, -p].  Every
// product bf16*fp32 or fp32*fp32 is exact in float64, so fma and mul+add agree
// and the ids are bit-reproducible.
//
// Sort: least-significant-digit counting sort per (b, h) segment over chunks
// of 256 tokens (one work group).  Each pass is histogram -> exclusive scan
// over (digit, chunk) -> stable scatter, with ranks inside a wave from
// ballot-based digit matching.  When positions are already ascending (the
// usual case) a single pass keyed by bucket suffices: the hash kernel then
// also writes the bucket histogram of its chunk, and the scatter copies the
// token rows (x and a companion tensor) to their sorted slots, so the whole
// call is three launches.  Otherwise four byte passes over the position come
// first.
#include <algorithm>

#include "scfa_device.hpp"
#include "scfa_internal.hpp"
#include "scfa_pipe.hpp"

namespace scfa {

constexpr int kHashThreads = kSortChunk;

// R ([H, d, half] float32) widened to float64 once per call and regrouped by
// column group: R64[h][g][k][c] = R[h][k][g*CG + c] for g*CG + c < half, else
// 0 ([H, cols/CG, d, CG] doubles in the workspace), so a group's values for
// consecutive coordinates are CG apart.
__global__ __launch_bounds__(256) void k_r_to_f64(const float *R, double *R64, int half, int cg_size, int d, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int c = i % cg_size;
  const int k = (i / cg_size) % d;
  const int hg = i / (cg_size * d);
  const int ngroups = (half + cg_size - 1) / cg_size;
  const int h = hg / ngroups, g = hg % ngroups;
  const int col = g * cg_size + c;
  R64[i] = col < half ? (double)R[((size_t)h * d + k) * half + col] : 0.0;
}

typedef __attribute__((address_space(4))) const double const_double;

// One thread per token, one 256-token sort chunk per work group.  R (float64)
// is read through the scalar unit: its addresses are uniform across the work
// group, so every product takes its R operand from scalar registers.  The x
// rows of the chunk pass through LDS in 64-byte column slabs (coalesced
// global loads, double-buffered, one barrier per slab; an 80-byte row pitch
// keeps each thread's 16-byte row reads conflict-free), because a thread
// reading its own row straight from memory touches one cache line per lane
// per load.  The CG column sums (8, 16 or 32 at a time) accumulate in float64
// over the coordinates in increasing order.  With `hist` set, the group also
// writes its chunk's bucket histogram.
constexpr int kSlabBytes = 64;
constexpr int kSlabPitch = 80;

// Coordinate k (0 .. 4*KP-1) of a slab row held as four 16-byte pieces.
template <bool F32, int KP>
__device__ __forceinline__ float slab_coord(const uint4 (&u)[4], int k) {
  const uint4 p = u[k / KP];
  const int e = k % KP;
  if (F32) {
    const uint32_t w = e == 0 ? p.x : e == 1 ? p.y : e == 2 ? p.z : p.w;
    return __uint_as_float(w);
  }
  const int wi = e >> 1;
  const uint32_t w = wi == 0 ? p.x : wi == 1 ? p.y : wi == 2 ? p.z : p.w;
  return bf16_bits_to_float((e & 1) ? (w >> 16) : (w & 0xffffu));
}

// R values of step st of a slab (see k_lsh_hash), from Rs = the column
// group's values for the slab's first coordinate: CG >= 16: coordinate
// st / (CG/16), columns 16*(st % (CG/16)) .. +15; CG == 8: coordinates 2*st
// and 2*st + 1, columns 0 .. 7.  All offsets are compile-time constants.
template <int CG>
__device__ __forceinline__ void load_r_step(double (&r)[16], const_double *Rs, int st) {
  const_double *p = Rs + (CG >= 16 ? (st / (CG / 16)) * CG + (st % (CG / 16)) * 16 : 16 * st);
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = p[i];
}

// Row of x that holds token t of sequence bh (see LshArgs::x_rows).
__device__ __forceinline__ size_t lsh_row(const LshArgs &a, int bh, int t) {
  return (size_t)bh * a.Tx + (a.x_rows ? min(max(a.x_rows[(size_t)bh * a.T + t], 0), a.Tx - 1) : t);
}

template <int D, int CG, bool F32>
__global__ __launch_bounds__(kHashThreads) void k_lsh_hash(LshArgs a, const double *R64, int32_t *hist, int nchunks) {
  constexpr int ES = F32 ? 4 : 2;          // bytes per coordinate
  constexpr int RB = D * ES;               // bytes per row
  constexpr int NS = RB / kSlabBytes;      // slabs per row
  constexpr int KP = 16 / ES;              // coordinates per 16-byte piece
  constexpr int PPS = kSlabBytes / 16;     // pieces per slab
  constexpr int NSS = PPS * KP * CG / 16;  // 16-value R steps per slab
  static_assert(kHashThreads == 256 && PPS == 4, "staging assumes 256 rows x 4 pieces");
  __shared__ __align__(16) unsigned char xs[2][kHashThreads * kSlabPitch];

  const int tid = threadIdx.x;
  const int bh = blockIdx.x / nchunks;
  const int tb = blockIdx.x % nchunks;
  const int h = bh % a.H;
  const int t0 = tb * kHashThreads;
  const int t = t0 + tid;
  const bool valid = t < a.T;
  const int half = a.nb / 2;
  const int ngroups = (half + CG - 1) / CG;
  const_double *Rh = (const_double *)(R64 + (size_t)h * ngroups * D * CG);
  const char *xb = static_cast<const char *>(a.x);

  // staging: this thread copies piece (tid & 3) of rows (tid >> 2) + 64j,
  // j = 0..3; rows past the end repeat the last row (never compared)
  const int sr = tid >> 2, sp = (tid & 3) * 16;
  const char *src0 = xb + lsh_row(a, bh, min(t0 + sr, a.T - 1)) * RB + sp;
  const char *src1 = xb + lsh_row(a, bh, min(t0 + sr + 64, a.T - 1)) * RB + sp;
  const char *src2 = xb + lsh_row(a, bh, min(t0 + sr + 128, a.T - 1)) * RB + sp;
  const char *src3 = xb + lsh_row(a, bh, min(t0 + sr + 192, a.T - 1)) * RB + sp;
  const int dst0 = sr * kSlabPitch + sp;  // rows +64j: + 64 * j * kSlabPitch
  uint4 st0 = *reinterpret_cast<const uint4 *>(src0);
  uint4 st1 = *reinterpret_cast<const uint4 *>(src1);
  uint4 st2 = *reinterpret_cast<const uint4 *>(src2);
  uint4 st3 = *reinterpret_cast<const uint4 *>(src3);

  double best = -INFINITY, worst = INFINITY;
  int besti = 0, worsti = 0;
  int buf = 0;
  for (int cg = 0; cg < half; cg += CG) {
    double acc[CG];
#pragma unroll
    for (int cc = 0; cc < CG; ++cc) acc[cc] = 0.0;
#pragma unroll 1
    for (int sl = 0; sl < NS; ++sl) {
      unsigned char *xbuf = xs[buf];
      *reinterpret_cast<uint4 *>(xbuf + dst0) = st0;
      *reinterpret_cast<uint4 *>(xbuf + dst0 + 64 * kSlabPitch) = st1;
      *reinterpret_cast<uint4 *>(xbuf + dst0 + 128 * kSlabPitch) = st2;
      *reinterpret_cast<uint4 *>(xbuf + dst0 + 192 * kSlabPitch) = st3;
      // next slab (wrapping to slab 0 for the next column group; one
      // redundant in-range load at the very end)
      const int nso = (sl + 1 < NS ? sl + 1 : 0) * kSlabBytes;
      st0 = *reinterpret_cast<const uint4 *>(src0 + nso);
      st1 = *reinterpret_cast<const uint4 *>(src1 + nso);
      st2 = *reinterpret_cast<const uint4 *>(src2 + nso);
      st3 = *reinterpret_cast<const uint4 *>(src3 + nso);
      __syncthreads();
      // this thread's row of the slab: PPS pieces of KP coordinates
      uint4 u[PPS];
#pragma unroll
      for (int pc = 0; pc < PPS; ++pc) u[pc] = *reinterpret_cast<const uint4 *>(xbuf + tid * kSlabPitch + pc * 16);
      // column group cg, first coordinate of the slab
      const_double *Rs = Rh + ((size_t)(cg / CG) * D + sl * PPS * KP) * CG;
      // The slab's products run in steps of 16 R values (one s_load_dwordx16
      // pair): one coordinate x 16 columns (CG 16), half a coordinate (CG 32)
      // or two coordinates x 8 columns (CG 8).  The next step's R values are
      // requested before the current step's FMAs so their latency overlaps.
      double rn[16];
      load_r_step<CG>(rn, Rs, 0);
#pragma unroll
      for (int st = 0; st < NSS; ++st) {
        double rc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) rc[i] = rn[i];
        if (st + 1 < NSS) load_r_step<CG>(rn, Rs, st + 1);
        if (CG >= 16) {
          const int k = st / (CG / 16), c0 = (st % (CG / 16)) * 16;
          const double xk = (double)slab_coord<F32, KP>(u, k);
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[c0 + i] = fma(xk, rc[i], acc[c0 + i]);
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const double xk = (double)slab_coord<F32, KP>(u, 2 * st + j);
#pragma unroll
            for (int i = 0; i < CG; ++i) acc[i] = fma(xk, rc[8 * j + i], acc[i]);
          }
        }
#if defined(__HIP_DEVICE_COMPILE__)
        __builtin_amdgcn_sched_barrier(0);  // bounds the R values live in scalar registers
#endif
      }
      buf ^= 1;
    }
    const int ncol = min(CG, half - cg);
#pragma unroll
    for (int cc = 0; cc < CG; ++cc) {
      if (cc < ncol) {
        const double p = acc[cc];
        if (p > best) {
          best = p;
          besti = cg + cc;
        }
        if (p < worst) {
          worst = p;
          worsti = cg + cc;
        }
      }
    }
  }
  const int bucket = best >= -worst ? besti : half + worsti;
  if (valid) a.hash[(size_t)bh * a.T + t] = bucket;
  if (hist) {
    // the staging buffers are free once every thread has read its last slab
    int *sh = reinterpret_cast<int *>(&xs[0][0]);
    __syncthreads();
    for (int i = tid; i < a.nb; i += kHashThreads) sh[i] = 0;
    __syncthreads();
    if (valid) atomicAdd(&sh[bucket], 1);
    __syncthreads();
    for (int i = tid; i < a.nb; i += kHashThreads) hist[((size_t)bh * a.nb + i) * nchunks + tb] = sh[i];
  }
}

template <int D, int CG>
static void launch_hash_cg(const LshArgs &a, const double *R64, int32_t *hist, int nchunks, unsigned grid,
                           hipStream_t s) {
  if (a.dtype == 1)
    hipLaunchKernelGGL((k_lsh_hash<D, CG, true>), dim3(grid), dim3(kHashThreads), 0, s, a, R64, hist, nchunks);
  else
    hipLaunchKernelGGL((k_lsh_hash<D, CG, false>), dim3(grid), dim3(kHashThreads), 0, s, a, R64, hist, nchunks);
}

template <int D>
static void launch_hash(const LshArgs &a, const double *R64, int32_t *hist, int nchunks, unsigned grid,
                        hipStream_t s) {
  const int half = a.nb / 2;
  const int g = lsh_col_group(a.nb);
  if (g == 8) launch_hash_cg<D, 8>(a, R64, hist, nchunks, grid, s);
  else if (g == 16) launch_hash_cg<D, 16>(a, R64, hist, nchunks, grid, s);
  else launch_hash_cg<D, 32>(a, R64, hist, nchunks, grid, s);
}

// ---------------------------------------------------------------------------
// Matrix-core projection with certified buckets (bf16 inputs).
//
// The bucket is defined by the float64 projection above.  For bf16 inputs it
// is computed on the matrix cores instead, and checked:
//  * R (float32) is split exactly into three bf16 terms, R = R1 + R2 + R3
//    (each term takes the next 8 significant bits), so x.R = x.R1 + x.R2 +
//    x.R3 with every bf16 x bf16 product exact in float32; the 3d products
//    of a column accumulate in float32 (v_mfma_f32_32x32x16_bf16).
//  * The float32 sum differs from the float64 one by at most
//    E = (3.25 d + 8) 2^-22 sum_k |x_k R_kc| <= (3.25 d + 8) 2^-22 |x| max_c |R_c|
//    (Cauchy-Schwarz): four times the worst case of rounding each of the
//    3d products' additions and the 3d/16 accumulator additions once in
//    float32, so it also covers truncating adders.
//  * If the largest of the 2*(nb/2) candidates [p, -p] exceeds the second by
//    more than 2E (plus a little for the float32 subtraction), its index is
//    the float64 bucket.  Otherwise (near ties, exact ties, non-finite
//    values) the token goes to a list that k_lsh_fallback recomputes in
//    float64, in the same order as k_lsh_hash.
// So the ids stay bit-exact, and only a small fraction of the tokens (those
// whose two best candidates are within about 1e-2 of each other at d = 128)
// pays for float64.
// ---------------------------------------------------------------------------

// R split into bf16 A-fragments: entry (h, ct, s, kk, lane) holds, for R
// column c = 32 ct + lane % 32, the 8 coordinates k = 16 kk + 8 (lane / 32) + j
// of term s (columns past nb/2 are zero).  Threads past the fragments compute
// the column norms; thread 0 clears the fallback counter.
template <int D>
__global__ __launch_bounds__(256) void k_r_split(const float *R, uint4 *Rf, float *colnorm, int32_t *fb_count, int H,
                                                 int half, int nct) {
  constexpr int d = D;
  const int kks = d / 16;
  const long long nfrag = (long long)H * nct * 3 * kks * 64;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i == 0) *fb_count = 0;
  if (i < nfrag) {
    const int lane = (int)(i % 64);
    const int kk = (int)((i / 64) % kks);
    const int sp = (int)((i / (64 * kks)) % 3);
    const int ct = (int)((i / (64 * kks * 3)) % nct);
    const int h = (int)(i / (64LL * kks * 3 * nct));
    const int c = 32 * ct + (lane & 31);
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      float t[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int k = 16 * kk + 8 * (lane >> 5) + j + q;
        const float r = c < half ? R[((size_t)h * d + k) * half + c] : 0.f;
        const float r1 = bf16_bits_to_float(pack_bf16x2(r, 0.f) & 0xffffu);
        const float rr = r - r1;  // exact
        const float r2 = bf16_bits_to_float(pack_bf16x2(rr, 0.f) & 0xffffu);
        const float r3 = rr - r2;  // exact, and at most 8 significant bits
        t[q] = sp == 0 ? r1 : sp == 1 ? r2 : r3;
      }
      w[j / 2] = pack_bf16x2(t[0], t[1]);
    }
    Rf[i] = make_uint4(w[0], w[1], w[2], w[3]);
  } else if (i < nfrag + (long long)H * half) {
    const long long j = i - nfrag;
    const int h = (int)(j / half), c = (int)(j % half);
    float rv[D];
#pragma unroll
    for (int k = 0; k < D; ++k) rv[k] = R[((size_t)h * D + k) * half + c];
    double ss = 0.0;
#pragma unroll
    for (int k = 0; k < D; ++k) ss = fma((double)rv[k], (double)rv[k], ss);
    colnorm[j] = (float)(sqrt(ss) * (1.0 + 1e-6));  // rounded up past float conversion and sqrt
  }
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Running top two of the projections of one token (largest and smallest p,
// with the index of the first) over the columns a lane sees.
// The two largest entries of z = [p, -p] are the largest |p_c| (as +p_c or
// -p_c, by its sign) and the largest |p_c| over the other columns (the
// opposite-sign entry of the winning column is <= 0 <= that), or -|p_c| when
// there is a single column.  So the kernel tracks the top two of |p| over
// distinct columns, the winner's column and its signed value.
struct Top2 {
  float a1, a2;  // largest |p|, second largest over the other columns
  float v1;      // signed p of the largest
  int i1;        // its column
};

__device__ __forceinline__ void top2_init(Top2 &t) {
  t.a1 = t.a2 = -INFINITY;
  t.v1 = 0.f;
  t.i1 = 0;
}

// Branch-free: the new second value is the median of (first, second, |v|); an
// equal value lands in the second slot (gap 0) and keeps the first column.
// Columns that take no part pass a = -inf.
__device__ __forceinline__ void top2_add(Top2 &t, float v, float a, int c) {
  const bool gt = a > t.a1;
  t.i1 = gt ? c : t.i1;
  t.v1 = gt ? v : t.v1;
  t.a2 = __builtin_amdgcn_fmed3f(t.a1, t.a2, a);
  t.a1 = fmaxf(t.a1, a);
}

// Merge with the state of lane l ^ 32 (the other 16 columns of each tile).
__device__ __forceinline__ void top2_merge_pair(Top2 &t) {
  const float oa1 = __shfl_xor(t.a1, 32, 64), oa2 = __shfl_xor(t.a2, 32, 64);
  const float ov1 = __shfl_xor(t.v1, 32, 64);
  const int oi1 = __shfl_xor(t.i1, 32, 64);
  // candidates are distinct columns; equal values end up in both slots (gap 0)
  if (oa1 > t.a1 || (oa1 == t.a1 && oi1 < t.i1)) {
    t.a2 = fmaxf(t.a1, oa2);
    t.a1 = oa1;
    t.i1 = oi1;
    t.v1 = ov1;
  } else {
    t.a2 = fmaxf(t.a2, oa1);
  }
}

template <int D>
__global__ __launch_bounds__(kHashThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_lsh_mfma(LshArgs a, const uint4 *Rf, const float *colnorm,
                                                           int32_t *hist, int nchunks) {
  constexpr int KK = D / 16;
  constexpr int NF = 3 * KK * 64;  // uint4 fragments of one 32-column tile of R
  constexpr int NP = NF / kHashThreads;
  constexpr float kErr = (3.25f * D + 8.f) * 0x1p-22f;
  __shared__ int sh[1024];     // bucket histogram of the chunk (nb <= 1024)
  __shared__ uint4 rt[2][NF];  // column tiles of R, double-buffered, shared by the group's waves
  const int bh = blockIdx.x / nchunks, tb = blockIdx.x % nchunks, h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int half = a.nb / 2, nct = (half + 31) / 32;
  const int t0 = tb * kHashThreads;

  // B operands: the wave's 64 tokens as two 32-token tiles (x rows, 8
  // coordinates per lane and k-step).
  const uint16_t *X = static_cast<const uint16_t *>(a.x);
  bf16x8 xf[2][KK];
  int tok[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    tok[n] = t0 + 64 * w + 32 * n + col;
    const bool tv = tok[n] < a.T;
    const size_t xr = tv ? lsh_row(a, bh, tok[n]) : 0;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      xf[n][kk] = as_bf16x8(tv ? ld16(X + xr * D + 16 * kk + 8 * hf) : make_uint4(0, 0, 0, 0));
  }
  // R tiles go straight from global memory to LDS (no registers held for them);
  // each wave copies 64 consecutive fragments per piece, lane l to slot 64 w + l.
  const uint4 *Rh = Rf + (size_t)h * nct * NF;
#pragma unroll
  for (int i = 0; i < NP; ++i) lds_copy16(Rh + tid + kHashThreads * i, &rt[0][64 * w + kHashThreads * i]);
  if (hist)
    for (int i = tid; i < a.nb; i += kHashThreads) sh[i] = 0;
  float rm = 0.f;
  for (int c = lane; c < half; c += 64) rm = fmaxf(rm, colnorm[(size_t)h * half + c]);
  rm = wave_max_f(rm);
  // each token's norm (this lane's half of the coordinates, then the pair)
  float xn[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    float ss = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const uint4 u = __builtin_bit_cast(uint4, xf[n][kk]);
      const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_bits_to_float(wd[e] & 0xffffu), hi = bf16_bits_to_float(wd[e] >> 16);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
    }
    xn[n] = sqrtf(pair_sum(ss)) * 1.0001f;  // rounded up past the float32 sum and sqrt
  }
  wait_vmem();  // the first R tile has landed in LDS
  __syncthreads();

  Top2 t2[2];
  top2_init(t2[0]);
  top2_init(t2[1]);
  for (int ct = 0; ct < nct; ++ct) {
    const int cb = ct & 1;
    const bool more = ct + 1 < nct;  // wave-uniform
    if (more) {  // the next tile into the other buffer, while this one is multiplied
      const uint4 *nsrc = Rh + (size_t)(ct + 1) * NF;
#pragma unroll
      for (int i = 0; i < NP; ++i) lds_copy16(nsrc + tid + kHashThreads * i, &rt[cb ^ 1][64 * w + kHashThreads * i]);
    }
    f32x16 acc0 = kZero16, acc1 = kZero16;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int sp = 0; sp < 3; ++sp) {
        const bf16x8 af = as_bf16x8(rt[cb][(sp * KK + kk) * 64 + lane]);
        acc0 = mfma32(af, xf[0][kk], acc0);
        acc1 = mfma32(af, xf[1][kk], acc1);
      }
    if (32 * (ct + 1) <= half) {  // whole tile in range (wave-uniform)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 32 * ct + 8 * (r >> 2) + 4 * hf + (r & 3);
        top2_add(t2[0], acc0[r], fabsf(acc0[r]), c);
        top2_add(t2[1], acc1[r], fabsf(acc1[r]), c);
      }
    } else {  // columns past nb/2 take no part
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 32 * ct + 8 * (r >> 2) + 4 * hf + (r & 3);
        top2_add(t2[0], acc0[r], c < half ? fabsf(acc0[r]) : -INFINITY, c);
        top2_add(t2[1], acc1[r], c < half ? fabsf(acc1[r]) : -INFINITY, c);
      }
    }
    if (more) wait_vmem();  // the next tile has landed before any wave reads it
    __syncthreads();
  }

  unsigned long long need[2];
  int bucket[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    Top2 &t = t2[n];
    top2_merge_pair(t);
    // top two of z = [p, -p]
    const float z1 = t.a1, z2 = fmaxf(t.a2, -t.a1);
    const int iz = t.v1 < 0.f ? half + t.i1 : t.i1;
    const float prod = xn[n] * rm;
    const float err = kErr * prod + 0x1p-100f * xn[n];
    const bool certified = prod < 1e37f && (z1 - z2) > 2.f * err + 0x1p-20f * (fabsf(z1) + fabsf(z2));
    const bool valid = tok[n] < a.T && hf == 0;
    bucket[n] = iz;
    need[n] = __ballot(valid && !certified);
    if (valid && certified) a.hash[(size_t)bh * a.T + tok[n]] = iz;
  }
  // uncertified tokens: append to the fallback list (one atomic per wave and tile)
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    if (need[n] == 0ull) continue;  // wave-uniform
    int base = 0;
    if (lane == 0) base = atomicAdd(a.fb_count, __popcll(need[n]));
    base = __shfl(base, 0, 64);
    const bool mine = (need[n] >> lane) & 1ull;
    if (mine) a.fb_list[base + __popcll(need[n] & ((1ull << lane) - 1ull))] = bh * a.T + tok[n];
  }
  if (hist) {
#pragma unroll
    for (int n = 0; n < 2; ++n)
      if (tok[n] < a.T && hf == 0 && !((need[n] >> lane) & 1ull)) atomicAdd(&sh[bucket[n]], 1);
    __syncthreads();
    for (int i = threadIdx.x; i < a.nb; i += kHashThreads) hist[((size_t)bh * a.nb + i) * nchunks + tb] = sh[i];
  }
}

// Float64 buckets of the listed tokens, one wave per token, lanes over the R
// columns: each lane loads its column of R (float32, widened exactly) in one
// batch and accumulates the projection over the coordinates in increasing
// order (as k_lsh_hash does), each coordinate of x broadcast by readlane;
// first max of p and first min of p are reduced over the wave.  The chunk
// histogram gets the token with an atomic add.  A fixed grid strides over the
// list.  (Each listed token reads all of R[h] through L2; the list is short.)
template <int D>
__global__ __launch_bounds__(256) void k_lsh_fallback(LshArgs a, int32_t *hist, int nchunks) {
  const int lane = threadIdx.x & 63;
  const int gw = (int)((blockIdx.x * 256 + threadIdx.x) >> 6), nw = (int)(gridDim.x * 4);
  const int n = *a.fb_count;
  const int half = a.nb / 2;
  for (int i = gw; i < n; i += nw) {
    const int e = a.fb_list[i];
    const int bh = e / a.T, t = e % a.T, h = bh % a.H;
    const uint16_t *xr = static_cast<const uint16_t *>(a.x) + lsh_row(a, bh, t) * D;
    // the row, one coordinate per lane (two for D = 128)
    const float x0 = bf16_bits_to_float(xr[lane]);
    const float x1 = D > 64 ? bf16_bits_to_float(xr[(64 + lane) % D]) : 0.f;
    double best = -INFINITY, worst = INFINITY;
    int besti = 0, worsti = 0;
    for (int c0 = 0; c0 < half; c0 += 64) {
      const int c = c0 + lane;
      const bool cv = c < half;
      const float *rp = a.R + (size_t)h * D * half + (cv ? c : half - 1);  // column c of R[h], stride half
      float rv[D];
#pragma unroll
      for (int k = 0; k < D; ++k) rv[k] = rp[(size_t)k * half];
#if defined(__HIP_DEVICE_COMPILE__)
      __builtin_amdgcn_sched_barrier(0);  // all loads in flight before the dependent chain
#endif
      double acc = 0.0;
#pragma unroll
      for (int k = 0; k < D; ++k) {
        const float xk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, k < 64 ? x0 : x1), k % 64));
        acc = fma((double)xk, (double)rv[k], acc);
      }
      if (cv) {
        if (acc > best) best = acc, besti = c;
        if (acc < worst) worst = acc, worsti = c;
      }
    }
    // first max / first min over the wave (lower index wins ties)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ob = __shfl_xor(best, o, 64), ow = __shfl_xor(worst, o, 64);
      const int obi = __shfl_xor(besti, o, 64), owi = __shfl_xor(worsti, o, 64);
      if (ob > best || (ob == best && obi < besti)) best = ob, besti = obi;
      if (ow < worst || (ow == worst && owi < worsti)) worst = ow, worsti = owi;
    }
    const int bucket = best >= -worst ? besti : half + worsti;
    if (lane == 0) {
      a.hash[e] = bucket;
      if (hist) atomicAdd(&hist[((size_t)bh * a.nb + bucket) * nchunks + t / kSortChunk], 1);
    }
  }
}

// ---------------------------------------------------------------------------
// One counting-sort pass.
// ---------------------------------------------------------------------------
struct SortPass {
  const int32_t *hash;     // [BH, T] bucket of each source row
  const int32_t *in_idx;   // current order: position of item (NULL => item index)
  const int32_t *in_src;   // current order: source row of item (NULL => item index)
  int32_t *out_idx, *out_src, *out_hash;  // out_hash only on the bucket pass
  int32_t *hist;           // [BH, nbins, nchunks]
  const int32_t *rowoff;   // [BH, nbins] digit offsets when hist holds per-row scans (two-level scan), else NULL
  int T, nbins, nbits, nchunks, shift, bucket_pass;
};

// Rows moved by the final pass: x[src] -> xs[slot], cmp[src] -> cs[slot].
struct RowCopy {
  const uint4 *x;
  uint4 *xs;
  const uint4 *cmp;
  uint4 *cs;
  int pieces;  // 16-byte pieces per row: 8, 16 or 32
};

__device__ __forceinline__ void item_at(const SortPass &p, size_t base, int pos, int &idx, int &src, int &digit) {
  idx = p.in_idx ? p.in_idx[base + pos] : pos;
  src = p.in_src ? p.in_src[base + pos] : pos;
  digit = p.bucket_pass ? p.hash[base + src] : ((unsigned)idx >> p.shift) & 255u;
}

__global__ __launch_bounds__(kSortChunk) void k_sort_hist(SortPass p) {
  extern __shared__ int sh[];
  const int bh = blockIdx.x / p.nchunks;
  const int chunk = blockIdx.x % p.nchunks;
  const size_t base = (size_t)bh * p.T;
  for (int i = threadIdx.x; i < p.nbins; i += kSortChunk) sh[i] = 0;
  __syncthreads();
  const int pos = chunk * kSortChunk + threadIdx.x;
  if (pos < p.T) {
    int idx, src, digit;
    item_at(p, base, pos, idx, src, digit);
    atomicAdd(&sh[digit], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < p.nbins; i += kSortChunk)
    p.hist[((size_t)bh * p.nbins + i) * p.nchunks + chunk] = sh[i];
}

// Exclusive scan of hist[bh] in (digit, chunk) order, in place.
__global__ __launch_bounds__(1024) void k_sort_scan(SortPass p) {
  __shared__ int part[1024];
  const int n = p.nbins * p.nchunks;
  int32_t *h = p.hist + (size_t)blockIdx.x * n;
  const int per = (n + 1023) / 1024;
  const int lo = min(n, (int)threadIdx.x * per), hi = min(n, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += h[i];
  part[threadIdx.x] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = threadIdx.x >= (unsigned)off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int run = part[threadIdx.x] - sum;
  for (int i = lo; i < hi; ++i) {
    const int v = h[i];
    h[i] = run;
    run += v;
  }
}

// Cooperative copy of a wave's 64 rows (row src of lane l -> row dst of lane
// l, skipped where dst < 0) for one or two matrices with P 16-byte pieces per
// row: each instruction moves 64 / P rows, P lanes per row.  Eight
// instructions' loads are issued before their stores so that their latencies
// overlap (the compiler may not move a load above a store to a buffer that
// might alias it).
template <int P, bool TWO>
__device__ __forceinline__ void copy_rows(const uint4 *x0_, uint4 *y0_, const uint4 *x1_, uint4 *y1_, size_t base,
                                          int src, int dst, int lane) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 *x0 = reinterpret_cast<const u32x4 *>(x0_), *x1 = reinterpret_cast<const u32x4 *>(x1_);
  u32x4 *y0 = reinterpret_cast<u32x4 *>(y0_), *y1 = reinterpret_cast<u32x4 *>(y1_);
  constexpr int PER_IT = 64 / P;
  constexpr int NB = 8;
  const int piece = lane % P;
#pragma unroll
  for (int it0 = 0; it0 < P; it0 += NB) {
    int ss[NB], sl[NB];
    u32x4 v0[NB], v1[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int tok = (it0 + j) * PER_IT + lane / P;
      ss[j] = __shfl(src, tok, 64);
      sl[j] = __shfl(dst, tok, 64);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      v0[j] = x0[(base + ss[j]) * P + piece];
      if (TWO) v1[j] = x1[(base + ss[j]) * P + piece];
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (sl[j] >= 0) {
        y0[(base + sl[j]) * P + piece] = v0[j];
        if (TWO) y1[(base + sl[j]) * P + piece] = v1[j];
      }
  }
}

// Two-level scan for long segments (nbins * nchunks entries per (b, h)).
// First level: one work group per (b, h, digit) row; exclusive scan of the
// row's chunk counts in place, row total to tot.
__global__ __launch_bounds__(256) void k_sort_scan_rows(SortPass p, int32_t *tot) {
  __shared__ int part[256];
  int32_t *row = p.hist + (size_t)blockIdx.x * p.nchunks;
  const int tid = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < p.nchunks; base += 256) {
    const int i = base + tid;
    const int v = i < p.nchunks ? row[i] : 0;
    part[tid] = v;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int u = tid >= off ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += u;
      __syncthreads();
    }
    if (i < p.nchunks) row[i] = carry + part[tid] - v;
    carry += part[255];
    __syncthreads();
  }
  if (tid == 0) tot[blockIdx.x] = carry;
}

// Second level: per (b, h), exclusive scan of the row totals over the digits
// (nbins <= 1024).
__global__ __launch_bounds__(1024) void k_sort_scan_tot(SortPass p, const int32_t *tot, int32_t *rowoff) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const size_t base = (size_t)blockIdx.x * p.nbins;
  const int v = tid < p.nbins ? tot[base + tid] : 0;
  part[tid] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int u = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += u;
    __syncthreads();
  }
  if (tid < p.nbins) rowoff[base + tid] = part[tid] - v;
}

// Stable scatter of one 256-token chunk; wave w owns tokens 64w .. 64w+63.
// P = rc.pieces (16-byte pieces per row).
template <int P>
__global__ __launch_bounds__(kSortChunk) void k_sort_scatter(SortPass p, RowCopy rc) {
  extern __shared__ int cnt[];  // [4][nbins]
  const int bh = blockIdx.x / p.nchunks;
  const int chunk = blockIdx.x % p.nchunks;
  const size_t base = (size_t)bh * p.T;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int pos = chunk * kSortChunk + threadIdx.x;
  const bool valid = pos < p.T;
  int idx = 0, src = 0, digit = 0;
  if (valid) item_at(p, base, pos, idx, src, digit);

  for (int i = threadIdx.x; i < 4 * p.nbins; i += kSortChunk) cnt[i] = 0;
  unsigned long long peers = __ballot(valid);
  for (int b = 0; b < p.nbits; ++b) {
    const bool bit = (digit >> b) & 1;
    const unsigned long long m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  const int rank = __popcll(peers & ((1ull << lane) - 1ull));
  __syncthreads();
  if (valid && rank == 0) cnt[w * p.nbins + digit] = __popcll(peers);
  __syncthreads();
  int slot = 0;
  if (valid) {
    slot = p.hist[((size_t)bh * p.nbins + digit) * p.nchunks + chunk] + rank;
    if (p.rowoff) slot += p.rowoff[(size_t)bh * p.nbins + digit];
    for (int ww = 0; ww < w; ++ww) slot += cnt[ww * p.nbins + digit];
    p.out_idx[base + slot] = idx;
    p.out_src[base + slot] = src;
    if (p.bucket_pass) p.out_hash[base + slot] = digit;
  }
  const int dst_slot = valid ? slot : -1;  // src is 0 (a real row) on padding lanes
  if (rc.xs && rc.cs) copy_rows<P, true>(rc.x, rc.xs, rc.cmp, rc.cs, base, src, dst_slot, lane);
  else if (rc.xs) copy_rows<P, false>(rc.x, rc.xs, nullptr, nullptr, base, src, dst_slot, lane);
  else if (rc.cs) copy_rows<P, false>(rc.cmp, rc.cs, nullptr, nullptr, base, src, dst_slot, lane);
}

// Segments longer than this use the two-level scan.
constexpr int kScanOneGroup = 32768;

static hipError_t run_pass(SortPass p, const RowCopy &rc, int BH, bool with_hist, int32_t *scan_tmp, hipStream_t s) {
  const unsigned grid = (unsigned)(BH * p.nchunks);
  hipError_t e;
  if (with_hist) {
    hipLaunchKernelGGL(k_sort_hist, dim3(grid), dim3(kSortChunk), p.nbins * sizeof(int), s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((long long)p.nbins * p.nchunks > kScanOneGroup) {
    int32_t *tot = scan_tmp, *rowoff = scan_tmp + (size_t)BH * p.nbins;
    hipLaunchKernelGGL(k_sort_scan_rows, dim3((unsigned)(BH * p.nbins)), dim3(256), 0, s, p, tot);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_sort_scan_tot, dim3((unsigned)BH), dim3(1024), 0, s, p, tot, rowoff);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    p.rowoff = rowoff;
  } else {
    p.rowoff = nullptr;
    hipLaunchKernelGGL(k_sort_scan, dim3((unsigned)BH), dim3(1024), 0, s, p);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = 4 * p.nbins * sizeof(int);
  if (rc.pieces == 32) hipLaunchKernelGGL(k_sort_scatter<32>, dim3(grid), dim3(kSortChunk), lds, s, p, rc);
  else if (rc.pieces == 16) hipLaunchKernelGGL(k_sort_scatter<16>, dim3(grid), dim3(kSortChunk), lds, s, p, rc);
  else hipLaunchKernelGGL(k_sort_scatter<8>, dim3(grid), dim3(kSortChunk), lds, s, p, rc);
  return hipGetLastError();
}

hipError_t launch_lsh_bucket_sort(const LshArgs &a, hipStream_t s) {
  const int BH = a.B * a.H;
  if (BH == 0 || a.T == 0) return hipSuccess;
  const int nchunks = sort_chunks(a.T);
  const bool idx_passes = a.idx != nullptr && !a.idx_ascending;
  const unsigned hgrid = (unsigned)(BH * nchunks);
  int32_t *fused_hist = idx_passes ? nullptr : a.hist;
  hipError_t e;
  if (a.dtype == 0) {
    // bf16: matrix-core projection, certified; float64 for the rest
    const int half = a.nb / 2, nct = lsh_col_tiles(a.nb);
    const long long nsplit = (long long)a.H * nct * 3 * (a.d / 16) * 64 + (long long)a.H * half;
    const unsigned sgrid = (unsigned)((nsplit + 255) / 256);
    uint4 *Rf = static_cast<uint4 *>(a.Rf);
    if (a.d == 64) hipLaunchKernelGGL(k_r_split<64>, dim3(sgrid), dim3(256), 0, s, a.R, Rf, a.colnorm, a.fb_count, a.H, half, nct);
    else hipLaunchKernelGGL(k_r_split<128>, dim3(sgrid), dim3(256), 0, s, a.R, Rf, a.colnorm, a.fb_count, a.H, half, nct);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.d == 64) hipLaunchKernelGGL(k_lsh_mfma<64>, dim3(hgrid), dim3(kHashThreads), 0, s, a, Rf, a.colnorm, fused_hist, nchunks);
    else hipLaunchKernelGGL(k_lsh_mfma<128>, dim3(hgrid), dim3(kHashThreads), 0, s, a, Rf, a.colnorm, fused_hist, nchunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const long long ntok = (long long)BH * a.T;
    const unsigned fgrid = (unsigned)std::min<long long>(2048, (ntok + 3) / 4);
    if (a.d == 64) hipLaunchKernelGGL(k_lsh_fallback<64>, dim3(fgrid), dim3(256), 0, s, a, fused_hist, nchunks);
    else hipLaunchKernelGGL(k_lsh_fallback<128>, dim3(fgrid), dim3(256), 0, s, a, fused_hist, nchunks);
  } else {
    const int nr = a.H * a.d * lsh_r64_cols(a.nb);
    hipLaunchKernelGGL(k_r_to_f64, dim3((unsigned)((nr + 255) / 256)), dim3(256), 0, s, a.R, a.R64, a.nb / 2,
                       lsh_col_group(a.nb), a.d, nr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.d == 64) launch_hash<64>(a, a.R64, fused_hist, nchunks, hgrid, s);
    else launch_hash<128>(a, a.R64, fused_hist, nchunks, hgrid, s);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  SortPass p{};
  p.hash = a.hash;
  p.hist = a.hist;
  p.T = a.T;
  p.nchunks = nchunks;
  p.in_idx = a.idx;
  p.in_src = nullptr;
  const RowCopy none{nullptr, nullptr, nullptr, nullptr, 8};
  int buf = 0;
  if (idx_passes) {
    for (int shift = 0; shift < 32; shift += 8) {
      p.nbins = 256;
      p.nbits = 8;
      p.shift = shift;
      p.bucket_pass = 0;
      p.out_idx = a.tmp_idx[buf];
      p.out_src = a.tmp_src[buf];
      p.out_hash = nullptr;
      e = run_pass(p, none, BH, true, a.scan_tmp, s);
      if (e != hipSuccess) return e;
      p.in_idx = a.tmp_idx[buf];
      p.in_src = a.tmp_src[buf];
      buf ^= 1;
    }
  }
  p.nbins = a.nb;
  p.nbits = 1;
  while ((1 << p.nbits) < a.nb) ++p.nbits;
  p.shift = 0;
  p.bucket_pass = 1;
  p.out_idx = a.idx_sorted;
  p.out_src = a.perm;
  p.out_hash = a.hash_sorted;
  RowCopy rc{static_cast<const uint4 *>(a.x), static_cast<uint4 *>(a.x_sorted),
             static_cast<const uint4 *>(a.companion), static_cast<uint4 *>(a.companion_sorted),
             a.d * (a.dtype == 1 ? 4 : 2) / 16};
  return run_pass(p, rc, BH, idx_passes, a.scan_tmp, s);
}

}  // namespace scfa
