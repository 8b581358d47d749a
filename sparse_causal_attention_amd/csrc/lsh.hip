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
#include "scfa_device.hpp"
#include "scfa_internal.hpp"

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
  const char *xb = static_cast<const char *>(a.x) + (size_t)bh * a.T * RB;

  // staging: this thread copies piece (tid & 3) of rows (tid >> 2) + 64j,
  // j = 0..3; rows past the end repeat the last row (never compared)
  const int sr = tid >> 2, sp = (tid & 3) * 16;
  const char *src0 = xb + (size_t)min(t0 + sr, a.T - 1) * RB + sp;
  const char *src1 = xb + (size_t)min(t0 + sr + 64, a.T - 1) * RB + sp;
  const char *src2 = xb + (size_t)min(t0 + sr + 128, a.T - 1) * RB + sp;
  const char *src3 = xb + (size_t)min(t0 + sr + 192, a.T - 1) * RB + sp;
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
// One counting-sort pass.
// ---------------------------------------------------------------------------
struct SortPass {
  const int32_t *hash;     // [BH, T] bucket of each source row
  const int32_t *in_idx;   // current order: position of item (NULL => item index)
  const int32_t *in_src;   // current order: source row of item (NULL => item index)
  int32_t *out_idx, *out_src, *out_hash;  // out_hash only on the bucket pass
  int32_t *hist;           // [BH, nbins, nchunks]
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

static hipError_t run_pass(const SortPass &p, const RowCopy &rc, int BH, bool with_hist, hipStream_t s) {
  const unsigned grid = (unsigned)(BH * p.nchunks);
  hipError_t e;
  if (with_hist) {
    hipLaunchKernelGGL(k_sort_hist, dim3(grid), dim3(kSortChunk), p.nbins * sizeof(int), s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_sort_scan, dim3((unsigned)BH), dim3(1024), 0, s, p);
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
  const int nr = a.H * a.d * lsh_r64_cols(a.nb);
  hipLaunchKernelGGL(k_r_to_f64, dim3((unsigned)((nr + 255) / 256)), dim3(256), 0, s, a.R, a.R64, a.nb / 2,
                     lsh_col_group(a.nb), a.d, nr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.d == 64) launch_hash<64>(a, a.R64, fused_hist, nchunks, hgrid, s);
  else launch_hash<128>(a, a.R64, fused_hist, nchunks, hgrid, s);
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
      e = run_pass(p, none, BH, true, s);
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
  return run_pass(p, rc, BH, idx_passes, s);
}

}  // namespace scfa
