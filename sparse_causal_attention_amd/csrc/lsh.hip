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
// Sort: least-significant-digit counting sort per (b, h) segment.  Each pass
// is histogram -> exclusive scan over (digit, chunk) -> stable scatter, with
// ranks inside a wave from ballot-based digit matching.  When positions are
// already ascending (the usual case) a single pass keyed by bucket suffices;
// otherwise four byte passes over the position come first.
#include "scfa_device.hpp"
#include "scfa_internal.hpp"

namespace scfa {

constexpr int kHashThreads = 256;

// One thread per token.  R's columns are processed in groups of CG (8, 16 or
// 32, the smallest that covers nb/2 or 32): the group is widened to float64
// once into LDS and every thread accumulates CG float64 sums over the
// coordinates in increasing order, eight coordinates (one 16-byte load of x)
// per step.
template <int D, int CG, bool F32>
__global__ __launch_bounds__(kHashThreads) void k_lsh_hash(LshArgs a) {
  __shared__ __attribute__((aligned(16))) double sR[D * CG];
  const int nblk = (a.T + kHashThreads - 1) / kHashThreads;
  const int bh = blockIdx.x / nblk;
  const int tb = blockIdx.x % nblk;
  const int h = bh % a.H;
  const int t = tb * kHashThreads + threadIdx.x;
  const bool valid = t < a.T;
  const int half = a.nb / 2;
  const float *R = a.R + (size_t)h * D * half;
  const size_t row = (size_t)bh * a.T + (valid ? t : 0);

  double best = -INFINITY, worst = INFINITY;
  int besti = 0, worsti = 0;
  for (int cg = 0; cg < half; cg += CG) {
    const int ncol = min(CG, half - cg);
    __syncthreads();
    for (int i = threadIdx.x; i < D * CG; i += kHashThreads) {
      const int k = i / CG, cc = i % CG;
      sR[i] = cc < ncol ? (double)R[(size_t)k * half + cg + cc] : 0.0;
    }
    __syncthreads();
    double acc[CG];
#pragma unroll
    for (int cc = 0; cc < CG; ++cc) acc[cc] = 0.0;
#pragma unroll 1
    for (int k0 = 0; k0 < D; k0 += 8) {
      float xv[8];
      if (F32) {
        const float *X = static_cast<const float *>(a.x) + row * D + k0;
        const float4 v0 = valid ? *reinterpret_cast<const float4 *>(X) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 v1 = valid ? *reinterpret_cast<const float4 *>(X + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        xv[0] = v0.x; xv[1] = v0.y; xv[2] = v0.z; xv[3] = v0.w;
        xv[4] = v1.x; xv[5] = v1.y; xv[6] = v1.z; xv[7] = v1.w;
      } else {
        const uint16_t *X = static_cast<const uint16_t *>(a.x) + row * D + k0;
        const uint4 v = valid ? ld16(X) : make_uint4(0, 0, 0, 0);
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xv[2 * e] = bf16_bits_to_float(wv[e] & 0xffffu);
          xv[2 * e + 1] = bf16_bits_to_float(wv[e] >> 16);
        }
      }
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const double xk = (double)xv[kk];
        const double2 *r2 = reinterpret_cast<const double2 *>(sR + (k0 + kk) * CG);
#pragma unroll
        for (int c2 = 0; c2 < CG / 2; ++c2) {
          const double2 r = r2[c2];
          acc[2 * c2] = fma(xk, r.x, acc[2 * c2]);
          acc[2 * c2 + 1] = fma(xk, r.y, acc[2 * c2 + 1]);
        }
      }
    }
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
  if (valid) a.hash[(size_t)bh * a.T + t] = best >= -worst ? besti : half + worsti;
}

template <int D, int CG>
static void launch_hash_cg(const LshArgs &a, unsigned grid, hipStream_t s) {
  if (a.dtype == 1) hipLaunchKernelGGL((k_lsh_hash<D, CG, true>), dim3(grid), dim3(kHashThreads), 0, s, a);
  else hipLaunchKernelGGL((k_lsh_hash<D, CG, false>), dim3(grid), dim3(kHashThreads), 0, s, a);
}

template <int D>
static void launch_hash(const LshArgs &a, unsigned grid, hipStream_t s) {
  const int half = a.nb / 2;
  if (half <= 8) launch_hash_cg<D, 8>(a, grid, s);
  else if (half <= 16) launch_hash_cg<D, 16>(a, grid, s);
  else launch_hash_cg<D, 32>(a, grid, s);
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

__device__ __forceinline__ void item_at(const SortPass &p, size_t base, int pos, int &idx, int &src, int &digit) {
  idx = p.in_idx ? p.in_idx[base + pos] : pos;
  src = p.in_src ? p.in_src[base + pos] : pos;
  digit = p.bucket_pass ? p.hash[base + src] : ((unsigned)idx >> p.shift) & 255u;
}

__global__ __launch_bounds__(256) void k_sort_hist(SortPass p) {
  extern __shared__ int sh[];
  const int bh = blockIdx.x / p.nchunks;
  const int chunk = blockIdx.x % p.nchunks;
  const size_t base = (size_t)bh * p.T;
  for (int i = threadIdx.x; i < p.nbins; i += 256) sh[i] = 0;
  __syncthreads();
  const int c1 = min(p.T, (chunk + 1) * kSortChunk);
  for (int pos = chunk * kSortChunk + threadIdx.x; pos < c1; pos += 256) {
    int idx, src, digit;
    item_at(p, base, pos, idx, src, digit);
    atomicAdd(&sh[digit], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < p.nbins; i += 256)
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

__global__ __launch_bounds__(256) void k_sort_scatter(SortPass p) {
  extern __shared__ int cnt[];  // [4][nbins]
  const int bh = blockIdx.x / p.nchunks;
  const int chunk = blockIdx.x % p.nchunks;
  const size_t base = (size_t)bh * p.T;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c0 = chunk * kSortChunk, c1 = min(p.T, c0 + kSortChunk);
  constexpr int kPerWave = kSortChunk / 4;
  const int w0 = c0 + w * kPerWave, w1 = min(c1, w0 + kPerWave);

  for (int i = threadIdx.x; i < 4 * p.nbins; i += 256) cnt[i] = 0;
  __syncthreads();
  for (int pos = w0 + lane; pos < w1; pos += 64) {
    int idx, src, digit;
    item_at(p, base, pos, idx, src, digit);
    atomicAdd(&cnt[w * p.nbins + digit], 1);
  }
  __syncthreads();
  for (int dgt = threadIdx.x; dgt < p.nbins; dgt += 256) {
    int run = p.hist[((size_t)bh * p.nbins + dgt) * p.nchunks + chunk];
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const int tmp = cnt[ww * p.nbins + dgt];
      cnt[ww * p.nbins + dgt] = run;
      run += tmp;
    }
  }
  __syncthreads();
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int r0 = w0; r0 < w1; r0 += 64) {
    const int pos = r0 + lane;
    const bool valid = pos < w1;
    int idx = 0, src = 0, digit = 0;
    if (valid) item_at(p, base, pos, idx, src, digit);
    unsigned long long peers = __ballot(valid);
    for (int b = 0; b < p.nbits; ++b) {
      const bool bit = (digit >> b) & 1;
      const unsigned long long m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lt);
    const bool leader = valid && rank == 0;
    int slot = 0;
    if (valid) slot = cnt[w * p.nbins + digit];
    if (leader) cnt[w * p.nbins + digit] = slot + __popcll(peers);
    if (valid) {
      const size_t o = base + slot + rank;
      p.out_idx[o] = idx;
      p.out_src[o] = src;
      if (p.bucket_pass) p.out_hash[o] = digit;
    }
  }
}

// x_sorted[s] = x[perm[s]] (and the companion tensor), 16-byte pieces.
__global__ __launch_bounds__(256) void k_gather_rows(const int32_t *perm, const uint4 *x, uint4 *xs, const uint4 *cmp,
                                                     uint4 *cs, int T, int cpr, int rows_per_block) {
  const int nblk = (T + rows_per_block - 1) / rows_per_block;
  const int bh = blockIdx.x / nblk;
  const int r0 = (blockIdx.x % nblk) * rows_per_block;
  const size_t base = (size_t)bh * T;
  for (int i = threadIdx.x; i < rows_per_block * cpr; i += 256) {
    const int r = r0 + i / cpr, c = i % cpr;
    if (r >= T) break;
    const int src = perm[base + r];
    if (xs) xs[(base + r) * cpr + c] = x[(base + src) * cpr + c];
    if (cs) cs[(base + r) * cpr + c] = cmp[(base + src) * cpr + c];
  }
}

static hipError_t run_pass(const SortPass &p, int BH, hipStream_t s) {
  const unsigned grid = (unsigned)(BH * p.nchunks);
  hipLaunchKernelGGL(k_sort_hist, dim3(grid), dim3(256), p.nbins * sizeof(int), s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sort_scan, dim3((unsigned)BH), dim3(1024), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sort_scatter, dim3(grid), dim3(256), 4 * p.nbins * sizeof(int), s, p);
  return hipGetLastError();
}

hipError_t launch_lsh_bucket_sort(const LshArgs &a, hipStream_t s) {
  const int BH = a.B * a.H;
  if (BH == 0 || a.T == 0) return hipSuccess;
  const unsigned hgrid = (unsigned)(BH * ((a.T + kHashThreads - 1) / kHashThreads));
  if (a.d == 64) launch_hash<64>(a, hgrid, s);
  else launch_hash<128>(a, hgrid, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const bool idx_passes = a.idx != nullptr && !a.idx_ascending;
  SortPass p{};
  p.hash = a.hash;
  p.hist = a.hist;
  p.T = a.T;
  p.nchunks = sort_chunks(a.T);
  p.in_idx = a.idx;
  p.in_src = nullptr;
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
      e = run_pass(p, BH, s);
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
  e = run_pass(p, BH, s);
  if (e != hipSuccess) return e;

  if (a.x_sorted || a.companion_sorted) {
    const int esz = a.dtype == 1 ? 4 : 2;
    const int cpr = a.d * esz / 16;
    const int rows_per_block = 2048 / cpr;
    const unsigned grid = (unsigned)(BH * ((a.T + rows_per_block - 1) / rows_per_block));
    hipLaunchKernelGGL(k_gather_rows, dim3(grid), dim3(256), 0, s, a.perm, static_cast<const uint4 *>(a.x),
                       static_cast<uint4 *>(a.x_sorted), static_cast<const uint4 *>(a.companion),
                       static_cast<uint4 *>(a.companion_sorted), a.T, cpr, rows_per_block);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace scfa
