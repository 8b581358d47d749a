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
// after all its queries.  With per-block bucket segments (bucket, min
// position, max position) such tiles are dropped too: the tile is live iff
// some common bucket h has min key position <= max query position among the
// rows of bucket h.  Blocks with more than kMaxSegs distinct buckets keep the
// range test.  In QK-sparse mode the range test is already exact.
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
  // Bucket segments.  A block holds at most 128 rows: two per lane.
  const int lane = threadIdx.x;
  bool rem0 = r0 + lane < r1, rem1 = r0 + 64 + lane < r1;
  int h0 = 0, i0 = 0, h1 = 0, i1 = 0;
  if (rem0) h0 = hs[(size_t)bh * T + r0 + lane], i0 = idx[r0 + lane];
  if (rem1) h1 = hs[(size_t)bh * T + r0 + 64 + lane], i1 = idx[r0 + 64 + lane];
  int rec[3 * kMaxSegs];
  int nseg = 0;
#pragma unroll
  for (int sg = 0; sg < kMaxSegs; ++sg) {
    rec[3 * sg] = rec[3 * sg + 1] = rec[3 * sg + 2] = 0;
    if (__ballot(rem0 || rem1) == 0ull) continue;  // wave-uniform
    const int h = wave_min(min(rem0 ? h0 : INT32_MAX, rem1 ? h1 : INT32_MAX));
    const bool in0 = rem0 && h0 == h, in1 = rem1 && h1 == h;
    rec[3 * sg] = h;
    rec[3 * sg + 1] = wave_min(min(in0 ? i0 : INT32_MAX, in1 ? i1 : INT32_MAX));
    rec[3 * sg + 2] = wave_max(max(in0 ? i0 : INT32_MIN, in1 ? i1 : INT32_MIN));
    rem0 = rem0 && !in0;
    rem1 = rem1 && !in1;
    ++nseg;
  }
  const bool over = __ballot(rem0 || rem1) != 0ull;  // more than kMaxSegs buckets: count -1, records 0
  if (lane == 0) {
    int4 *out = reinterpret_cast<int4 *>(segs + ((size_t)bh * (isq ? a.nq : a.nk) + blk) * kSegInts);
    out[0] = make_int4(over ? -1 : nseg, 0, 0, 0);
#pragma unroll
    for (int sg = 0; sg < kMaxSegs; ++sg)
      out[1 + sg] = over ? make_int4(0, 0, 0, 0) : make_int4(rec[3 * sg], rec[3 * sg + 1], rec[3 * sg + 2], 0);
  }
}

// Exact test for a tile that passed the range test: some bucket common to the
// two blocks has a key at or before one of its queries.
__device__ __forceinline__ bool segs_admit(const int4 (&q)[1 + kMaxSegs], const int4 (&k)[1 + kMaxSegs]) {
  if (q[0].x < 0 || k[0].x < 0) return true;  // too many buckets: keep the range test's answer
  bool any = false;
#pragma unroll
  for (int s = 0; s < kMaxSegs; ++s)
#pragma unroll
    for (int t = 0; t < kMaxSegs; ++t)
      any = any || (s < q[0].x && t < k[0].x && q[1 + s].x == k[1 + t].x && k[1 + t].y <= q[1 + s].z);
  return any;
}

__global__ __launch_bounds__(64) void k_build_lists(MetaArgs a, int hash_mode, int with_cols) {
  const int nrow = a.nq + (with_cols ? a.nk : 0);
  const int bh = blockIdx.x / nrow;
  const int r = blockIdx.x % nrow;
  const bool is_row = r < a.nq;
  const int lane = threadIdx.x;
  const int4 *qst = reinterpret_cast<const int4 *>(a.q_stats) + (size_t)bh * a.nq;
  const int4 *kst = reinterpret_cast<const int4 *>(a.k_stats) + (size_t)bh * a.nk;
  const bool exact = hash_mode && a.q_segs != nullptr;
  const int4 *qsg = exact ? reinterpret_cast<const int4 *>(a.q_segs) + (size_t)bh * a.nq * (1 + kMaxSegs) : nullptr;
  const int4 *ksg = exact ? reinterpret_cast<const int4 *>(a.k_segs) + (size_t)bh * a.nk * (1 + kMaxSegs) : nullptr;
  int n_other;
  int32_t *list;
  int32_t *cnt_out;
  int4 mine;
  int4 mseg[1 + kMaxSegs];
  const int4 *other_seg;
  if (is_row) {
    n_other = a.nk;
    mine = qst[r];
    list = a.row_list + ((size_t)bh * a.nq + r) * a.nk;
    cnt_out = a.row_cnt + (size_t)bh * a.nq + r;
    other_seg = ksg;
    if (exact)
#pragma unroll
      for (int i = 0; i <= kMaxSegs; ++i) mseg[i] = qsg[(size_t)r * (1 + kMaxSegs) + i];
  } else {
    const int j = r - a.nq;
    n_other = a.nq;
    mine = kst[j];
    list = a.col_list + ((size_t)bh * a.nk + j) * a.nq;
    cnt_out = a.col_cnt + (size_t)bh * a.nk + j;
    other_seg = qsg;
    if (exact)
#pragma unroll
      for (int i = 0; i <= kMaxSegs; ++i) mseg[i] = ksg[(size_t)j * (1 + kMaxSegs) + i];
  }
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
      if (exact && live) {
        int4 oseg[1 + kMaxSegs];
#pragma unroll
        for (int i = 0; i <= kMaxSegs; ++i) oseg[i] = other_seg[(size_t)o * (1 + kMaxSegs) + i];
        live = is_row ? segs_admit(mseg, oseg) : segs_admit(oseg, mseg);
      }
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
