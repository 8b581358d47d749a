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
// zeros for them and a scatter drops them.
#include "scfa_device.hpp"
#include "scfa_internal.hpp"

namespace scfa {

constexpr int kRowThreads = 256;

// dst[bh, i, :] = src[bh, index[bh, i], :] for i < Td (zeros when the index
// is outside [0, Ts)).  ppr = 16-byte pieces per row.
__global__ __launch_bounds__(kRowThreads) void k_gather_rows(const uint4 *src, const int32_t *index, uint4 *dst,
                                                              int Ts, int Td, int ppr, long long total) {
  const long long stride = (long long)gridDim.x * kRowThreads;
  for (long long p = (long long)blockIdx.x * kRowThreads + threadIdx.x; p < total; p += stride) {
    const long long row = p / ppr;
    const int piece = (int)(p - row * ppr);
    const long long bh = row / Td;
    const int j = index[row];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j >= 0 && j < Ts) v = src[(bh * Ts + j) * ppr + piece];
    dst[p] = v;
  }
}

// dst[bh, index[bh, i], :] = src[bh, i, :] for i < Ts (rows whose index is
// outside [0, Td) are dropped).
__global__ __launch_bounds__(kRowThreads) void k_scatter_rows(const uint4 *src, const int32_t *index, uint4 *dst,
                                                               int Ts, int Td, int ppr, long long total) {
  const long long stride = (long long)gridDim.x * kRowThreads;
  for (long long p = (long long)blockIdx.x * kRowThreads + threadIdx.x; p < total; p += stride) {
    const long long row = p / ppr;
    const int piece = (int)(p - row * ppr);
    const long long bh = row / Ts;
    const int j = index[row];
    if (j >= 0 && j < Td) dst[(bh * Td + j) * ppr + piece] = src[p];
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

hipError_t launch_gather_rows(const RowArgs &r, hipStream_t s) {
  const long long total = (long long)r.BH * r.Td * r.ppr;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gather_rows, dim3(row_grid(total)), dim3(kRowThreads), 0, s,
                     static_cast<const uint4 *>(r.src), r.index, static_cast<uint4 *>(r.dst), r.Ts, r.Td, r.ppr,
                     total);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(const RowArgs &r, bool zero_fill, hipStream_t s) {
  if (zero_fill) {
    const long long n = (long long)r.BH * r.Td * r.ppr;
    if (n > 0) {
      hipLaunchKernelGGL(k_zero_pieces, dim3(row_grid(n)), dim3(kRowThreads), 0, s, static_cast<uint4 *>(r.dst), n);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  const long long total = (long long)r.BH * r.Ts * r.ppr;
  if (total == 0 || r.Td == 0) return hipSuccess;
  hipLaunchKernelGGL(k_scatter_rows, dim3(row_grid(total)), dim3(kRowThreads), 0, s,
                     static_cast<const uint4 *>(r.src), r.index, static_cast<uint4 *>(r.dst), r.Ts, r.Td, r.ppr,
                     total);
  return hipGetLastError();
}

}  // namespace scfa
