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
  int T = isq ? a.Tq : a.Tk;
  size_t base = (size_t)bh * T;
  const int32_t *off = isq ? a.q_off : a.k_off;
  if (off) {  // packed ragged heads: this head's rows and length (blocks past it stay empty), clamped
    const long long tot = isq ? a.q_total : a.k_total;  // into the packed rows as in varlen_head
    const long long b0 = min(max((long long)off[bh], 0ll), tot);
    base = (size_t)b0;
    T = (int)min(max((long long)off[bh + 1] - b0, 0ll), min((long long)T, tot - b0));
  }
  const int32_t *idx = (isq ? a.q_idx : a.k_idx) + base;
  const int32_t *hs = isq ? a.q_hash : a.k_hash;
  if (hs) hs += base;
  const int r0 = blk * a.block;
  const int r1 = min(r0 + a.block, T);
  // A block holds at most 128 rows: two per lane, loaded once for both the
  // statistics and the bucket records.
  const int lane = threadIdx.x;
  bool rem0 = r0 + lane < r1, rem1 = r0 + 64 + lane < r1;
  int h0 = 0, i0 = 0, h1 = 0, i1 = 0;
  if (rem0) {
    i0 = idx[r0 + lane];
    if (hs) h0 = hs[r0 + lane];
  }
  if (rem1) {
    i1 = idx[r0 + 64 + lane];
    if (hs) h1 = hs[r0 + 64 + lane];
  }
  const int mn = wave_min(min(rem0 ? i0 : INT32_MAX, rem1 ? i1 : INT32_MAX));
  const int mx = wave_max(max(rem0 ? i0 : INT32_MIN, rem1 ? i1 : INT32_MIN));
  int hmn = 0, hmx = 0;
  if (hs) {
    hmn = wave_min(min(rem0 ? h0 : INT32_MAX, rem1 ? h1 : INT32_MAX));
    hmx = wave_max(max(rem0 ? h0 : INT32_MIN, rem1 ? h1 : INT32_MIN));
  }
  if (lane == 0) {
    int32_t *out = (isq ? a.q_stats + ((size_t)bh * a.nq + blk) * 4 : a.k_stats + ((size_t)bh * a.nk + blk) * 4);
    *reinterpret_cast<int4 *>(out) = make_int4(mn, mx, hmn, hmx);
  }
  int32_t *segs = isq ? a.q_segs : a.k_segs;
  if (segs == nullptr || hs == nullptr) return;
  // Bucket segments: the smallest remaining bucket id, then the min and max
  // position of its rows, until every row is taken (one record per distinct
  // bucket, at most `block`).
  const int nblk_side = isq ? a.nq : a.nk;
  int4 *out = reinterpret_cast<int4 *>(segs) + ((size_t)bh * nblk_side + blk) * a.block;
  int nseg = 0;
  if (hmn == hmx) {  // one bucket (or no rows): its record is the block's statistics
    nseg = r0 < r1 ? 1 : 0;
    if (lane == 0 && nseg) out[0] = make_int4(hmn, mn, mx, 0);
    rem0 = rem1 = false;
  }
  int h = hmn;  // the smallest remaining bucket id (the first is the block's minimum)
  while (__ballot(rem0 || rem1) != 0ull) {  // wave-uniform; each pass takes at least one row
    if (nseg > 0) h = wave_min(min(rem0 ? h0 : INT32_MAX, rem1 ? h1 : INT32_MAX));
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
// mine_is_q says which side holds the queries.  o0 and o1 are other[0] and
// other[1], already loaded (most blocks hold one or two buckets).
__device__ __forceinline__ bool segs_admit(const int4 *mine, int n_mine, const int4 *other, int n_other, int4 o0,
                                           int4 o1, bool mine_is_q) {
  int a = 0, b = 0;
  while (a < n_mine && b < n_other) {
    const int4 m = mine[a], o = b == 0 ? o0 : (b == 1 ? o1 : other[b]);
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
  // Partner statistics are read kPass x 64 at a time, all loads issued before
  // any is used; the first batch goes out before this block's own records, so
  // a list of up to kPass x 64 partners costs one round trip.
  constexpr int kPass = 4;
  const int n_part = is_row ? a.nk : a.nq;
  const int4 *ost = is_row ? kst : qst;
  const int32_t *onseg = is_row ? a.k_nseg : a.q_nseg;  // partners' record counts (exact rule)
  if (exact) onseg += (size_t)bh * n_part;
  int4 st[kPass];
  int on[kPass];
  auto load_pass = [&](int base0) {
#pragma unroll
    for (int u = 0; u < kPass; ++u) {
      const int o = base0 + 64 * u + lane;
      st[u] = o < n_part ? ost[o] : make_int4(0, 0, 0, 0);
      on[u] = exact && o < n_part ? onseg[o] : 0;
    }
  };
  load_pass(0);
  int n_other;
  int32_t *list;
  int32_t *cnt_out;
  int4 mine;
  const int4 *other_seg = nullptr;  // partner blocks' records, `block` slots each
  int n_mine = 0;
  if (is_row) {
    n_other = a.nk;
    mine = qst[r];
    list = a.row_list + ((size_t)bh * a.nq + r) * a.nk;
    cnt_out = a.row_cnt + (size_t)bh * a.nq + r;
    if (exact) {
      const int4 *src = reinterpret_cast<const int4 *>(a.q_segs) + ((size_t)bh * a.nq + r) * a.block;
      n_mine = min(a.q_nseg[(size_t)bh * a.nq + r], a.block);
      for (int t = lane; t < a.block; t += 64) mine_seg[t] = src[t];  // every slot (no wait for the count)
      other_seg = reinterpret_cast<const int4 *>(a.k_segs) + (size_t)bh * a.nk * a.block;
    }
  } else {
    const int j = r - a.nq;
    n_other = a.nq;
    mine = kst[j];
    list = a.col_list + ((size_t)bh * a.nk + j) * a.nq;
    cnt_out = a.col_cnt + (size_t)bh * a.nk + j;
    if (exact) {
      const int4 *src = reinterpret_cast<const int4 *>(a.k_segs) + ((size_t)bh * a.nk + j) * a.block;
      n_mine = min(a.k_nseg[(size_t)bh * a.nk + j], a.block);
      for (int t = lane; t < a.block; t += 64) mine_seg[t] = src[t];  // every slot (no wait for the count)
      other_seg = reinterpret_cast<const int4 *>(a.q_segs) + (size_t)bh * a.nq * a.block;
    }
  }
  __syncthreads();  // mine_seg written by the wave's lanes, read by all
  int count = 0;
  for (int base0 = 0; base0 < n_other; base0 += kPass * 64) {
    if (base0 > 0) load_pass(base0);
    // The range test for every pass first; the first two records of each
    // partner that needs the exact test are then loaded together.
    bool live[kPass], free[kPass], need[kPass];
    int4 rec0[kPass], rec1[kPass];
#pragma unroll
    for (int u = 0; u < kPass; ++u) {
      const int o = base0 + 64 * u + lane;
      live[u] = free[u] = need[u] = false;
      if (o < n_other) {
        const int4 qs = is_row ? mine : st[u];
        const int4 ks = is_row ? st[u] : mine;
        live[u] = qs.y >= ks.x;
        free[u] = ks.y <= qs.x;
        if (hash_mode) {
          live[u] = live[u] && qs.w >= ks.z && qs.z <= ks.w;
          free[u] = free[u] && qs.z == qs.w && ks.z == ks.w && qs.z == ks.z;
        }
        // With one bucket on each side the range test is already exact.
        need[u] = exact && live[u] && !(qs.z == qs.w && ks.z == ks.w);
      }
      rec0[u] = rec1[u] = make_int4(0, 0, 0, 0);
      if (need[u]) {
        const int4 *os = other_seg + (size_t)o * a.block;
        const int no = min(on[u], a.block);
        if (no > 0) rec0[u] = os[0];
        if (no > 1) rec1[u] = os[1];
      }
    }
#pragma unroll
    for (int u = 0; u < kPass; ++u) {
      const int base = base0 + 64 * u;
      if (base >= n_other) break;  // wave-uniform
      const int o = base + lane;
      bool lv = live[u];
      if (need[u])
        lv = segs_admit(mine_seg, n_mine, other_seg + (size_t)o * a.block, min(on[u], a.block), rec0[u], rec1[u],
                        is_row);
      const unsigned long long m = __ballot(lv);
      if (lv) {
        const int pos = count + __popcll(m & ((1ull << lane) - 1ull));
        list[pos] = o | (free[u] ? (int)0x80000000u : 0);
      }
      count += __popcll(m);
    }
  }
  if (lane == 0) *cnt_out = count;
}

// ---------------------------------------------------------------------------
// Tile slots: a numbering of the live tiles for the backward's stored dS.
// Slots follow the column lists: key block c (over all heads, c = bh*nk + j)
// owns slots col_base[c] .. col_base[c] + count - 1, in its list order, so the
// dK/dV kernel writes a key block's tiles to consecutive slots.  The dQ
// kernel walks row lists; row_slot gives, for each row-list entry, the slot of
// that tile (col_base of its key block + the rank of query block i in that
// block's column list).
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 1024;
constexpr int kScanItems = 16;

__device__ __forceinline__ int clamp_count(int c, int hi) { return min(max(c, 0), hi); }

// Exclusive scan of the (clamped) counts over all heads; base[n] is the total.
__global__ __launch_bounds__(kScanThreads) void k_count_scan(const int32_t *cnt, int n, int cap, int32_t *base) {
  __shared__ int wave_tot[kScanThreads / 64];
  __shared__ int carry_s;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  if (t == 0) carry_s = 0;
  __syncthreads();
  for (int b0 = 0; b0 < n; b0 += kScanThreads * kScanItems) {
    const int first = b0 + t * kScanItems;
    int v[kScanItems];
    int sum = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
      v[k] = first + k < n ? clamp_count(cnt[first + k], cap) : 0;
      sum += v[k];
    }
    // inclusive scan of the thread sums within the wave, then across waves
    int inc = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane == 63) wave_tot[w] = inc;
    __syncthreads();
    int wave_off = 0;
    for (int k = 0; k < w; ++k) wave_off += wave_tot[k];
    int run = carry_s + wave_off + inc - sum;  // exclusive prefix of this thread's first item
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
      if (first + k < n) base[first + k] = run;
      run += v[k];
    }
    __syncthreads();  // every thread has read carry_s and wave_tot
    if (t == kScanThreads - 1) carry_s = run;
    __syncthreads();
  }
  if (t == 0) base[n] = carry_s;
}

// row_slot[bh, i, t] = slot of the tile (i, j) named by row-list entry t
// (-1 if key block j's column list does not hold i, which lists from the
// builder never do).
__global__ __launch_bounds__(64) void k_row_slots(const int32_t *row_cnt, const int32_t *row_list,
                                                  const int32_t *col_cnt, const int32_t *col_list,
                                                  const int32_t *col_base, int32_t *row_slot, int nq, int nk) {
  const int bh = blockIdx.x / nq;
  const int i = blockIdx.x % nq;
  const size_t rrow = ((size_t)bh * nq + i) * nk;
  const int n = clamp_count(row_cnt[(size_t)bh * nq + i], nk);
  for (int t = threadIdx.x; t < n; t += 64) {
    const int j = row_list[rrow + t] & 0x7fffffff;
    int slot = -1;
    if (j < nk) {
      const int32_t *cl = col_list + ((size_t)bh * nk + j) * nq;
      const int m = clamp_count(col_cnt[(size_t)bh * nk + j], nq);
      int lo = 0, hi = m;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((cl[mid] & 0x7fffffff) < i) lo = mid + 1;
        else hi = mid;
      }
      if (lo < m && (cl[lo] & 0x7fffffff) == i) slot = col_base[(size_t)bh * nk + j] + lo;
    }
    row_slot[rrow + t] = slot;
  }
}

hipError_t launch_tile_slots(const int32_t *row_cnt, const int32_t *row_list, const int32_t *col_cnt,
                             const int32_t *col_list, int BH, int nq, int nk, int32_t *col_base, int32_t *row_slot,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_count_scan, dim3(1), dim3(kScanThreads), 0, s, col_cnt, BH * nk, nq, col_base);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || BH * nq == 0) return e;
  hipLaunchKernelGGL(k_row_slots, dim3((unsigned)(BH * nq)), dim3(64), 0, s, row_cnt, row_list, col_cnt, col_list,
                     col_base, row_slot, nq, nk);
  return hipGetLastError();
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
