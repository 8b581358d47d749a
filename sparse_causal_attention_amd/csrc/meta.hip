// Block metadata and live-tile lists.
//
// Tile pruning rules of SCFA (deep-paper.org summary of arXiv 2306.01160,
// "SCFA solution > 1. QK-Sparse" rule 1 and "2. Hash-Sparse" rules 1-2):
// a tile (query block i, key block j) is skipped when every query precedes
// every key, and in Hash-sparse mode when the blocks' buckets cannot match.
// The bucket test uses the blocks' [min, max] bucket ranges (interval
// overlap); the element mask inside the tile is exact, so this only decides
// which tiles are visited.
//
// Exact variant (Hash-sparse): a tile that passes the range test can still
// hold no valid pair, when every bucket the two blocks share has all its keys
// after all its queries.  Each block's distinct buckets are listed with the
// min and max position of their rows ("segments", as many as the block has
// buckets); the tile is live iff some common bucket h has min key position
// <= max query position among the rows of bucket h, which is exactly "the
// tile holds a valid pair".  In QK-sparse mode the range test is already
// exact.
//
// Two launches: block statistics (one wave per block), then one wave per list
// row that tests 64 partner blocks per step and compacts the live ones in
// ascending order with a ballot + popcount prefix.
#include "scfa_device.hpp"
#include "scfa_internal.hpp"

namespace scfa {

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

__global__ __launch_bounds__(64) void k_block_stats(MetaArgs a) {
  const int nblk = a.nq + a.nk;
  const int bh = blockIdx.x / nblk;
  const int b = blockIdx.x % nblk;
  const bool isq = b < a.nq;
  const int blk = isq ? b : b - a.nq;
  const int T = isq ? a.Tq : a.Tk;
  const int32_t *idx = (isq ? a.q_idx : a.k_idx) + (size_t)bh * T;
  const int32_t *hs = isq ? a.q_hash : a.k_hash;
  const int r0 = blk * a.block;
  const int r1 = min(r0 + a.block, T);
  int mn = INT32_MAX, mx = INT32_MIN, hmn = INT32_MAX, hmx = INT32_MIN;
  for (int r = r0 + (int)threadIdx.x; r < r1; r += 64) {
    const int v = idx[r];
    mn = min(mn, v);
    mx = max(mx, v);
    if (hs) {
      const int h = hs[(size_t)bh * T + r];
      hmn = min(hmn, h);
      hmx = max(hmx, h);
    }
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (hs) {
    hmn = wave_min(hmn);
    hmx = wave_max(hmx);
  } else {
    hmn = hmx = 0;
  }
  if (threadIdx.x == 0) {
    int32_t *out = (isq ? a.q_stats + ((size_t)bh * a.nq + blk) * 4 : a.k_stats + ((size_t)bh * a.nk + blk) * 4);
    *reinterpret_cast<int4 *>(out) = make_int4(mn, mx, hmn, hmx);
  }
  int32_t *segs = isq ? a.q_segs : a.k_segs;
  if (segs == nullptr || hs == nullptr) return;
  // Bucket segments: the smallest remaining bucket id, then the min and max
  // position of its rows, until every row is taken (one record per distinct
  // bucket, at most `block`).  A block holds at most 128 rows: two per lane.
  const int lane = threadIdx.x;
  bool rem0 = r0 + lane < r1, rem1 = r0 + 64 + lane < r1;
  int h0 = 0, i0 = 0, h1 = 0, i1 = 0;
  if (rem0) h0 = hs[(size_t)bh * T + r0 + lane], i0 = idx[r0 + lane];
  if (rem1) h1 = hs[(size_t)bh * T + r0 + 64 + lane], i1 = idx[r0 + 64 + lane];
  const int nblk_side = isq ? a.nq : a.nk;
  int4 *out = reinterpret_cast<int4 *>(segs) + ((size_t)bh * nblk_side + blk) * a.block;
  int nseg = 0;
  while (__ballot(rem0 || rem1) != 0ull) {  // wave-uniform; each pass takes at least one row
    const int h = wave_min(min(rem0 ? h0 : INT32_MAX, rem1 ? h1 : INT32_MAX));
    const bool in0 = rem0 && h0 == h, in1 = rem1 && h1 == h;
    const int mn2 = wave_min(min(in0 ? i0 : INT32_MAX, in1 ? i1 : INT32_MAX));
    const int mx2 = wave_max(max(in0 ? i0 : INT32_MIN, in1 ? i1 : INT32_MIN));
    if (lane == 0) out[nseg] = make_int4(h, mn2, mx2, 0);
    rem0 = rem0 && !in0;
    rem1 = rem1 && !in1;
    ++nseg;
  }
  if (lane == 0) (isq ? a.q_nseg : a.k_nseg)[(size_t)bh * nblk_side + blk] = nseg;
}

// Exact test for a tile that passed the range test: some bucket common to the
// two blocks has a key at or before one of its queries.  Both record lists are
// in ascending bucket order, so one merge pass finds the common buckets.
// `mine` (in LDS) belongs to the list's own block, `other` to the partner;
// mine_is_q says which side holds the queries.
__device__ __forceinline__ bool segs_admit(const int4 *mine, int n_mine, const int4 *other, int n_other,
                                           bool mine_is_q) {
  int a = 0, b = 0;
  while (a < n_mine && b < n_other) {
    const int4 m = mine[a], o = other[b];
    if (m.x < o.x) {
      ++a;
    } else if (m.x > o.x) {
      ++b;
    } else {
      if (mine_is_q ? o.y <= m.z : m.y <= o.z) return true;  // min key position <= max query position
      ++a;
      ++b;
    }
  }
  return false;
}

__global__ __launch_bounds__(64) void k_build_lists(MetaArgs a, int hash_mode, int with_cols) {
  __shared__ int4 mine_seg[128];  // this list's block's segments (block <= 128 rows)
  const int nrow = a.nq + (with_cols ? a.nk : 0);
  const int bh = blockIdx.x / nrow;
  const int r = blockIdx.x % nrow;
  const bool is_row = r < a.nq;
  const int lane = threadIdx.x;
  const int4 *qst = reinterpret_cast<const int4 *>(a.q_stats) + (size_t)bh * a.nq;
  const int4 *kst = reinterpret_cast<const int4 *>(a.k_stats) + (size_t)bh * a.nk;
  const bool exact = hash_mode && a.q_segs != nullptr;
  int n_other;
  int32_t *list;
  int32_t *cnt_out;
  int4 mine;
  const int4 *other_seg = nullptr;  // partner blocks' records, `block` slots each
  const int32_t *other_n = nullptr;
  int n_mine = 0;
  if (is_row) {
    n_other = a.nk;
    mine = qst[r];
    list = a.row_list + ((size_t)bh * a.nq + r) * a.nk;
    cnt_out = a.row_cnt + (size_t)bh * a.nq + r;
    if (exact) {
      const int4 *src = reinterpret_cast<const int4 *>(a.q_segs) + ((size_t)bh * a.nq + r) * a.block;
      n_mine = a.q_nseg[(size_t)bh * a.nq + r];
      for (int t = lane; t < n_mine; t += 64) mine_seg[t] = src[t];
      other_seg = reinterpret_cast<const int4 *>(a.k_segs) + (size_t)bh * a.nk * a.block;
      other_n = a.k_nseg + (size_t)bh * a.nk;
    }
  } else {
    const int j = r - a.nq;
    n_other = a.nq;
    mine = kst[j];
    list = a.col_list + ((size_t)bh * a.nk + j) * a.nq;
    cnt_out = a.col_cnt + (size_t)bh * a.nk + j;
    if (exact) {
      const int4 *src = reinterpret_cast<const int4 *>(a.k_segs) + ((size_t)bh * a.nk + j) * a.block;
      n_mine = a.k_nseg[(size_t)bh * a.nk + j];
      for (int t = lane; t < n_mine; t += 64) mine_seg[t] = src[t];
      other_seg = reinterpret_cast<const int4 *>(a.q_segs) + (size_t)bh * a.nq * a.block;
      other_n = a.q_nseg + (size_t)bh * a.nq;
    }
  }
  __syncthreads();  // mine_seg written by the wave's lanes, read by all
  int count = 0;
  for (int base = 0; base < n_other; base += 64) {
    const int o = base + lane;
    bool live = false, free = false;
    if (o < n_other) {
      const int4 qs = is_row ? mine : qst[o];
      const int4 ks = is_row ? kst[o] : mine;
      live = qs.y >= ks.x;
      free = ks.y <= qs.x;
      if (hash_mode) {
        live = live && qs.w >= ks.z && qs.z <= ks.w;
        free = free && qs.z == qs.w && ks.z == ks.w && qs.z == ks.z;
      }
      // With one bucket on each side the range test is already exact.
      if (exact && live && !(qs.z == qs.w && ks.z == ks.w))
        live = segs_admit(mine_seg, n_mine, other_seg + (size_t)o * a.block, other_n[o], is_row);
    }
    const unsigned long long m = __ballot(live);
    if (live) {
      const int pos = count + __popcll(m & ((1ull << lane) - 1ull));
      list[pos] = o | (free ? (int)0x80000000u : 0);
    }
    count += __popcll(m);
  }
  if (lane == 0) *cnt_out = count;
}

hipError_t launch_block_meta(const MetaArgs &a, bool with_cols, hipStream_t s) {
  const int hash_mode = a.q_hash != nullptr;
  if (a.nq + a.nk > 0) {
    hipLaunchKernelGGL(k_block_stats, dim3((unsigned)(a.BH * (a.nq + a.nk))), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nrow = a.nq + (with_cols ? a.nk : 0);
  if (nrow > 0) {
    hipLaunchKernelGGL(k_build_lists, dim3((unsigned)(a.BH * nrow)), dim3(64), 0, s, a, hash_mode,
                       with_cols ? 1 : 0);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace scfa
