// Row gather and scatter: the steps either side of the attention path.
//
// Tokens are dropped and the kept rows compacted before QK-sparse attention,
// or reordered by bucket before Hash-sparse attention, while every row keeps
// its original position (deep-paper.org summary of arXiv 2306.01160, "why
// dynamic sparsity breaks it" and "SCFA solution > 1. QK-Sparse": compact
// Q/K/V plus original positions).  Gather builds the compact / reordered
// tensors; scatter puts outputs and gradients back at their original rows.
//
// Pure data movement, bound by HBM bandwidth: each thread moves 16-byte
// pieces, consecutive threads consecutive pieces of a row, grid-stride.
// Index values outside the valid range never address memory: a gather writes
// zeros for them, a scatter and a row clear skip them.
#include "scfa_device.hpp"
#include "scfa_internal.hpp"

namespace scfa {

constexpr int kRowThreads = 256;

// One work group moves whole rows of one head (blockIdx.y = bh): 256 / ppr
// rows per step, ppr consecutive threads per row, grid-stride over the rows.
// PPR > 0 fixes the pieces per row at compile time (the row and piece of a
// thread are then a shift and a mask); PPR = 0 reads it from ppr_rt (at most
// 256).  No 64-bit division anywhere.
// Gather: dst[bh, i, :] = src[bh, index[bh, i], :] for i < Td (zeros when the
// index is outside [0, Ts)).
template <int PPR>
__global__ __launch_bounds__(kRowThreads) void k_gather_rows(const uint4 *src, const int32_t *index, uint4 *dst,
                                                              int Ts, int Td, int ppr_rt) {
  const int ppr = PPR > 0 ? PPR : ppr_rt;
  const int rpb = kRowThreads / ppr;  // rows per step of the group
  const int sub = (int)threadIdx.x / ppr, piece = (int)threadIdx.x - sub * ppr;
  if (sub >= rpb) return;
  const size_t bh = blockIdx.y;
  const uint4 *s = src + bh * (size_t)Ts * ppr;
  uint4 *d = dst + bh * (size_t)Td * ppr;
  const int32_t *ix = index + bh * (size_t)Td;
  for (long long i = (long long)blockIdx.x * rpb + sub; i < Td; i += (long long)gridDim.x * rpb) {
    const int j = ix[i];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j >= 0 && j < Ts) v = s[(size_t)j * ppr + piece];
    d[(size_t)i * ppr + piece] = v;
  }
}

// Scatter: dst[bh, index[bh, i], :] = src[bh, i, :] for i < Ts (rows whose
// index is outside [0, Td) are dropped).
template <int PPR>
__global__ __launch_bounds__(kRowThreads) void k_scatter_rows(const uint4 *src, const int32_t *index, uint4 *dst,
                                                               int Ts, int Td, int ppr_rt) {
  const int ppr = PPR > 0 ? PPR : ppr_rt;
  const int rpb = kRowThreads / ppr;
  const int sub = (int)threadIdx.x / ppr, piece = (int)threadIdx.x - sub * ppr;
  if (sub >= rpb) return;
  const size_t bh = blockIdx.y;
  const uint4 *s = src + bh * (size_t)Ts * ppr;
  uint4 *d = dst + bh * (size_t)Td * ppr;
  const int32_t *ix = index + bh * (size_t)Ts;
  for (long long i = (long long)blockIdx.x * rpb + sub; i < Ts; i += (long long)gridDim.x * rpb) {
    const int j = ix[i];
    if (j >= 0 && j < Td) d[(size_t)j * ppr + piece] = s[(size_t)i * ppr + piece];
  }
}

// Zero rows: dst[bh, index[bh, i], :] = 0 for i < Ts (indices outside [0, Td)
// are skipped; src is unused).  Clears the rows of dropped tokens in
// full-length outputs whose kept rows the attention kernels write directly.
template <int PPR>
__global__ __launch_bounds__(kRowThreads) void k_zero_rows(const uint4 *, const int32_t *index, uint4 *dst, int Ts,
                                                            int Td, int ppr_rt) {
  const int ppr = PPR > 0 ? PPR : ppr_rt;
  const int rpb = kRowThreads / ppr;
  const int sub = (int)threadIdx.x / ppr, piece = (int)threadIdx.x - sub * ppr;
  if (sub >= rpb) return;
  const size_t bh = blockIdx.y;
  uint4 *d = dst + bh * (size_t)Td * ppr;
  const int32_t *ix = index + bh * (size_t)Ts;
  // four rows per thread and pass, their indices loaded before any store (no load waits on a store)
  const long long stride = (long long)gridDim.x * rpb;
  for (long long i = (long long)blockIdx.x * rpb + sub; i < Ts; i += 4 * stride) {
    int j[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) j[u] = i + u * stride < Ts ? ix[i + u * stride] : -1;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j[u] >= 0 && j[u] < Td) d[(size_t)j[u] * ppr + piece] = make_uint4(0, 0, 0, 0);
  }
}

__global__ __launch_bounds__(kRowThreads) void k_zero_pieces(uint4 *dst, long long total) {
  const long long stride = (long long)gridDim.x * kRowThreads;
  for (long long p = (long long)blockIdx.x * kRowThreads + threadIdx.x; p < total; p += stride)
    dst[p] = make_uint4(0, 0, 0, 0);
}

static unsigned row_grid(long long total) {
  const long long g = (total + kRowThreads - 1) / kRowThreads;
  return (unsigned)(g < (1ll << 20) ? g : (1ll << 20));
}

// Grid of the row kernels: (row steps, BH), about 2^16 groups in all.
static dim3 rows_grid(int BH, int T, int ppr) {
  const long long steps = ((long long)T + kRowThreads / ppr - 1) / (kRowThreads / ppr);
  const long long cap = (1ll << 16) / BH + 1;
  return dim3((unsigned)(steps < cap ? steps : cap), (unsigned)BH);
}

#define SCFA_ROWS_LAUNCH(KERNEL, grid, r, Ts, Td)                                                              \
  do {                                                                                                        \
    const uint4 *src_ = static_cast<const uint4 *>((r).src);                                                  \
    uint4 *dst_ = static_cast<uint4 *>((r).dst);                                                              \
    switch ((r).ppr) {                                                                                        \
      case 8: hipLaunchKernelGGL(KERNEL<8>, grid, dim3(kRowThreads), 0, s, src_, (r).index, dst_, Ts, Td, 8); break;   \
      case 16: hipLaunchKernelGGL(KERNEL<16>, grid, dim3(kRowThreads), 0, s, src_, (r).index, dst_, Ts, Td, 16); break; \
      case 32: hipLaunchKernelGGL(KERNEL<32>, grid, dim3(kRowThreads), 0, s, src_, (r).index, dst_, Ts, Td, 32); break; \
      default: hipLaunchKernelGGL(KERNEL<0>, grid, dim3(kRowThreads), 0, s, src_, (r).index, dst_, Ts, Td, (r).ppr);    \
    }                                                                                                         \
  } while (0)

hipError_t launch_gather_rows(const RowArgs &r, hipStream_t s) {
  if ((long long)r.BH * r.Td * r.ppr == 0) return hipSuccess;
  if (r.ppr > kRowThreads || r.BH > 65535) return hipErrorInvalidValue;
  SCFA_ROWS_LAUNCH(k_gather_rows, rows_grid(r.BH, r.Td, r.ppr), r, r.Ts, r.Td);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(const RowArgs &r, bool zero_fill, hipStream_t s) {
  if (r.ppr > kRowThreads || r.BH > 65535) return hipErrorInvalidValue;
  if (zero_fill) {
    const long long n = (long long)r.BH * r.Td * r.ppr;
    if (n > 0) {
      hipLaunchKernelGGL(k_zero_pieces, dim3(row_grid(n)), dim3(kRowThreads), 0, s, static_cast<uint4 *>(r.dst), n);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if ((long long)r.BH * r.Ts * r.ppr == 0 || r.Td == 0) return hipSuccess;
  SCFA_ROWS_LAUNCH(k_scatter_rows, rows_grid(r.BH, r.Ts, r.ppr), r, r.Ts, r.Td);
  return hipGetLastError();
}

hipError_t launch_zero_rows(const RowArgs &r, hipStream_t s) {
  if ((long long)r.BH * r.Ts * r.ppr == 0 || r.Td == 0) return hipSuccess;
  if (r.ppr > kRowThreads || r.BH > 65535) return hipErrorInvalidValue;
  SCFA_ROWS_LAUNCH(k_zero_rows, rows_grid(r.BH, r.Ts, r.ppr), r, r.Ts, r.Td);
  return hipGetLastError();
}

}  // namespace scfa
