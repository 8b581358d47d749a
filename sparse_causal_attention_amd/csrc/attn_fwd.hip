// SCFA forward: tiled online-softmax attention over the live tiles of each
// query block, with the element mask on original positions (and buckets).
//
// deep-paper.org summary of arXiv 2306.01160: "SCFA solution > 1. QK-Sparse"
// (q_idx / k_idx inputs; skip acausal tiles; mask future tokens inside live
// tiles), "2. Hash-Sparse" (q_hash / k_hash; bucket pruning; mask on
// causality and bucket equality), "the rise of FlashAttention" (tiling keeps
// the softmax exact).
//
// bf16 kernel (gfx950 matrix cores).  One work group per (batch*head, query
// block of BS rows) with 2*BS/32 waves: each 32-query tile has two waves, one
// per half of every 64-key chunk, whose softmax states merge at the end.
// Each live key block is streamed through LDS in 64-key chunks: K row-major,
// V transposed.  The kernel computes S^T = K Q^T so that every lane owns ONE
// query column: the
// row max and row sum of the online softmax are in-lane except for a single
// exchange with lane l^32, the O^T accumulator rescale is in-lane, and the
// S^T registers feed the O^T += V^T P^T product directly as B operands.
//
// fp32 kernel: one thread per query, plain fp32 FMAs over 32-key LDS chunks.
#include "scfa_device.hpp"
#include "scfa_internal.hpp"
#include "scfa_pipe.hpp"

namespace scfa {

// Live list of a query block: the count, and for stored lists the first
// window of entries; entry t is read by tile_at.
template <int MODE, int BS>
__device__ __forceinline__ LiveList row_list(const AttnArgs &a, int bh, int qb) {
  LiveList r{0, 0, nullptr, 0, 0, 0};
  if (a.no_prune) {
    r.n = a.nk;
  } else if (MODE == kDense) {
    const int qmax = min((qb + 1) * BS, a.Tq) - 1;
    r.n = min(a.nk, qmax / BS + 1);
  } else {
    r.n = min(a.row_cnt[(size_t)bh * a.nq + qb], a.nk);  // malformed counts never overrun the row
    r.p = a.row_list + ((size_t)bh * a.nq + qb) * a.nk;
    r.lim = a.nk;
    list_window(r, 0);
  }
  return r;
}

// Key block of entry t and whether the whole tile is admissible (mask-free).
template <int MODE, int BS>
__device__ __forceinline__ void tile_at(const AttnArgs &a, LiveList &rl, int t, int qb, int &kb, bool &free) {
  if (a.no_prune) {
    kb = t;
    free = false;
  } else if (MODE == kDense) {
    kb = t;
    free = min((kb + 1) * BS, a.Tk) - 1 <= qb * BS;
  } else {
    const int e = list_entry(rl, t);
    kb = e & 0x7fffffff;
    free = e < 0;
  }
  if (a.force_mask) free = false;
}

// Position of one 64-key chunk in a row list.
struct ChunkPos {
  int t, ch, k0, kvalid;
  bool free;
};

// First usable chunk at or after entry t, chunk ch (entries naming a block
// outside the sequence and chunks past Tk are skipped).  Scalar code.
template <int MODE, int BS>
__device__ __forceinline__ bool find_chunk(const AttnArgs &a, LiveList &rl, int qb, int t, int ch, ChunkPos &out) {
  constexpr int NCH = BS / kChunk;
  for (; t < rl.n; ++t, ch = 0) {
    int kb;
    bool free;
    tile_at<MODE, BS>(a, rl, t, qb, kb, free);
    if (kb >= a.nk || ch >= NCH) continue;
    const int k0 = kb * BS + ch * kChunk;
    if (k0 >= a.Tk) continue;
    out.t = t;
    out.ch = ch;
    out.k0 = k0;
    out.kvalid = min(kChunk, a.Tk - k0);
    out.free = free;
    return true;
  }
  return false;
}

template <int D>
struct KVBuf {
  MatChunk<D> k, v;
  int idx[kChunk];
  int hash[kChunk];
};

template <int MODE, int D, int NW>
__device__ __forceinline__ void issue_kv(KVBuf<D> &b, const AttnArgs &a, const uint16_t *K, const uint16_t *V,
                                         int bh, const ChunkPos &c, const DmaOffsets<D, NW> &dof) {
  dma_matrix<D, NW>(b.k, K, c.k0, c.kvalid, dof);
  dma_matrix<D, NW>(b.v, V, c.k0, c.kvalid, dof);
  if (MODE != kDense && !(c.free && c.kvalid == kChunk)) {
    const int w = threadIdx.x >> 6;
    if (w == 0) dma_vec(b.idx, a.k_idx + (size_t)bh * a.Tk, c.k0, c.kvalid);
    if (MODE == kHash && w == NW - 1) dma_vec(b.hash, a.k_hash + (size_t)bh * a.Tk, c.k0, c.kvalid);
  }
}

// Lazy-rescale threshold of the online softmax, in log2 units: the reference
// max is only raised when a score exceeds it by more than this, so P <= 2^8.
constexpr float kRescaleLog2 = 8.f;

template <int MODE, int D, int NW>
__device__ __forceinline__ void issue_kv_rows(KVBuf<D> &b, const AttnArgs &a, const uint16_t *K, const uint16_t *V,
                                              int bh, const ChunkPos &c, const DmaRows<D, NW> &dr) {
  dma_matrix_rows<D, NW>(b.k, K, a.Tks, dr);
  dma_matrix_rows<D, NW>(b.v, V, a.Tks, dr);
  if (MODE != kDense && !(c.free && c.kvalid == kChunk)) {
    const int w = threadIdx.x >> 6;
    if (w == 0) dma_vec(b.idx, a.k_idx + (size_t)bh * a.Tk, c.k0, c.kvalid);
    if (MODE == kHash && w == NW - 1) dma_vec(b.hash, a.k_hash + (size_t)bh * a.Tk, c.k0, c.kvalid);
  }
}

// KROWS: K and V rows come through a.k_rows (the chunk copies read row
// k_rows[j] for chunk row j; the next chunk's indices are loaded one chunk
// ahead).  Q rows come through a.q_rows when it is set.
//
// 2*BS/32 waves per work group.  Wave w
// owns queries 32*(w % QW)..+31 (QW = BS/32) and keys 32*(w / QW)..+31 of
// every 64-key chunk, so each wave keeps its own online-softmax state over
// its half of the keys.  Twice the waves share each LDS chunk, so each wave
// needs about half the registers at the same LDS footprint: four waves per
// SIMD at d = 64 (128 VGPRs), no spills at d = 128.  At the end the second half's
// state (reference max, sum, O^T accumulator) goes through LDS and the
// first-half wave merges the two, as two partial softmaxes over disjoint key
// sets combine: m = max(m0, m1), l = l0 2^(m0-m) + l1 2^(m1-m) (log2 units),
// O = (acc0 2^(m0-m) + acc1 2^(m1-m)) / l.
//
// LB: block size of the lists (LB = BS, or LB = 2 BS: each LB-query block of
// the lists is run as two BS-query groups that walk the same list, every
// chunk masked on its own rows).  Each query sees the same chunks in the same
// order, split into the same key halves, as in one LB-query group, so the
// results are bit-identical; the smaller group runs at twice the groups per CU.
template <int MODE, int D, int BS, bool KROWS, int LB = BS>
__global__ __launch_bounds__(BS / 16 * 64) __attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 2))) void k_fwd_bf16_ks(
    AttnArgs a) {
  constexpr int QW = BS / 32;
  constexpr int NW = 2 * QW;
  static_assert(LB == BS || LB == 2 * BS, "a list block covers one or two query groups");
  __shared__ __attribute__((aligned(16))) KVBuf<D> sb[2];

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int ngroups = LB == BS ? a.nq : (a.Tq + BS - 1) / BS;  // query groups per head
  const int bh = wg / ngroups;
  const int qb = wg % ngroups;  // this group's queries: qb*BS ..
  const int qbl = qb / (LB / BS);  // and its row of the lists
  if (varlen_head(a, bh, 2) && qb * BS >= a.Tq) return;  // past this ragged head's queries
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int qw = w % QW, kh = w / QW;
  const int col = lane & 31, half = lane >> 5;
  const int qrow = qb * BS + 32 * qw + col;
  const bool qvalid = qrow < a.Tq;
  const uint16_t *Q = static_cast<const uint16_t *>(a.q) + (size_t)bh * a.Tqs * D;
  const uint16_t *K = static_cast<const uint16_t *>(a.k) + (size_t)bh * a.Tks * D;
  const uint16_t *V = static_cast<const uint16_t *>(a.v) + (size_t)bh * a.Tks * D;

  // Loads that depend only on this lane's own row go first: issued after the
  // list and chunk copies, a wait for them would also wait for those copies.
  int qsrc_raw = a.q_rows && qvalid ? a.q_rows[(size_t)bh * a.Tq + qrow] : qrow;  // clamped where used
  int my_idx = kIdxTailQ, my_hash = 0;
  if (qvalid) {
    my_idx = MODE == kDense ? qrow : a.q_idx[(size_t)bh * a.Tq + qrow];
    if (MODE == kHash) my_hash = a.q_hash[(size_t)bh * a.Tq + qrow];
  }
  LiveList rl = row_list<MODE, LB>(a, bh, qbl);
  // Consumed here, where the list window's wait already covers this older load;
  // first used after the chunk copies, its wait would also drain them.
  asm volatile("" : "+v"(qsrc_raw));
  const DmaOffsets<D, NW> dof = dma_offsets<D, NW>();
  const int32_t *krows = KROWS ? a.k_rows + (size_t)bh * a.Tk : nullptr;
  ChunkPos cur;
  bool have = find_chunk<MODE, LB>(a, rl, qbl, 0, 0, cur);
  DmaRows<D, NW> drn;  // KROWS: source rows of the next chunk to copy
  if (have) {
    if constexpr (KROWS) {
      dma_rows_load<D, NW>(drn, krows, cur.k0, cur.kvalid);
      issue_kv_rows<MODE, D, NW>(sb[0], a, K, V, bh, cur, drn);
    } else {
      issue_kv<MODE, D, NW>(sb[0], a, K, V, bh, cur, dof);
    }
  }
  ChunkPos nxt;
  bool have_next = false;
  if constexpr (KROWS) {
    have_next = have && find_chunk<MODE, LB>(a, rl, qbl, cur.t, cur.ch + 1, nxt);
    if (have_next) dma_rows_load<D, NW>(drn, krows, nxt.k0, nxt.kvalid);
  }
  const LaneOffsets<D> lo = lane_offsets<D>();

  const int qsrc = a.q_rows && qvalid ? min(max(qsrc_raw, 0), a.Tqs - 1) : qrow;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    qf[kk] = as_bf16x8(qvalid ? ld16(Q + (size_t)qsrc * D + 16 * kk + 8 * half) : make_uint4(0, 0, 0, 0));

  const float c = a.scale * kLog2e;
  float mref = -INFINITY, l = 0.f;
  f32x16 acc[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;

  int buf = 0;
  while (have) {
    ChunkPos nxt2;
    bool have_next2 = false;
    if constexpr (KROWS) have_next2 = have_next && find_chunk<MODE, LB>(a, rl, qbl, nxt.t, nxt.ch + 1, nxt2);
    else have_next = find_chunk<MODE, LB>(a, rl, qbl, cur.t, cur.ch + 1, nxt);
    wait_vmem();
    __syncthreads();
    if (have_next) {
      if constexpr (KROWS) issue_kv_rows<MODE, D, NW>(sb[buf ^ 1], a, K, V, bh, nxt, drn);
      else issue_kv<MODE, D, NW>(sb[buf ^ 1], a, K, V, bh, nxt, dof);
    }
    if constexpr (KROWS)
      if (have_next2) dma_rows_load<D, NW>(drn, krows, nxt2.k0, nxt2.kvalid);
    const KVBuf<D> &b = sb[buf];

    // S^T over this wave's 32 keys: all K fragments requested, then the chain.
    bf16x8 kfr[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) kfr[kk] = frag_rows<D>(b.k, lo, kh, kk);
    f32x16 s = mfma32(kfr[0], qf[0], kZero16);
#pragma unroll
    for (int kk = 1; kk < D / 16; ++kk) s = mfma32(kfr[kk], qf[kk], s);
    bf16x8 vfr[2][D / 32];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) vfr[t][mt] = frag_trans<D>(b.v, lo, mt, 2 * kh + t);
    if (cur.kvalid < kChunk)
      mask_tile_q<MODE, true>(s, b.idx, b.hash, 32 * kh, cur.k0, cur.kvalid, my_idx, my_hash, half, -INFINITY);
    else if (!cur.free)
      mask_tile_q<MODE, false>(s, b.idx, b.hash, 32 * kh, cur.k0, cur.kvalid, my_idx, my_hash, half, -INFINITY);

    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = pair_max(mx);
    const bool need = qvalid & (mx * c > mref * c + kRescaleLog2);
    if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
      const float m_new = fmaxf(mref, mx);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((mref - m_new) * c);
      if (__builtin_amdgcn_ballot_w64(mref != -INFINITY) != 0ull) {
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mt][r] *= alpha;
      }
      l *= alpha;
      mref = m_new;
    }
    const float mc = mref == -INFINITY ? 0.f : mref * c;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, -mc));
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const uint4 pk = c_regs_to_u4(s, t2);
      l = add_bf16x8(pk, l);
      const bf16x8 pb = as_bf16x8(pk);
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) acc[mt] = mfma32(vfr[t2][mt], pb, acc[mt]);
    }
    buf ^= 1;
    cur = nxt;
    have = have_next;
    if constexpr (KROWS) {
      nxt = nxt2;
      have_next = have_next2;
    }
  }

  // Merge the two key halves.  No copy is in flight here (the last chunk
  // issued none); the first barrier ends every wave's reads of the chunk
  // buffers before they are reused for the exchange.  The exchange goes in
  // rounds of QX query waves when all QW do not fit the buffers at once.
  float lt = pair_sum(l);
  // Lane-derived values of the epilogue are recomputed from an opaque copy of
  // the thread id, so none of them stays live across the chunk loop.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane_e = tid & 63, half_e = lane_e >> 5, qw_e = (tid >> 6) % QW;
  const int qrow_e = qb * BS + 32 * qw_e + (lane_e & 31);
  // The output row's index is loaded before the exchange below, whose barriers
  // wait only for LDS, so its latency overlaps the merge.
  int orow_raw = a.orig_rows && kh == 0 && qrow_e < a.Tq ? a.q_rows[(size_t)bh * a.Tq + qrow_e] : qrow_e;
  constexpr int XN = 2 + 16 * (D / 32);  // floats per lane: reference max, sum, accumulator
  constexpr int FIT = (int)(sizeof(sb) / (sizeof(float) * XN * 64));
  constexpr int QX = FIT >= QW ? QW : (FIT >= 2 ? 2 : 1);
  static_assert(FIT >= 1 && QW % QX == 0, "exchange does not fit the chunk buffers");
  float *xch = reinterpret_cast<float *>(sb) + (size_t)(qw_e % QX) * XN * 64 + lane_e;
  float m = mref;
#pragma unroll
  for (int round = 0; round < QW / QX; ++round) {
    const bool mine = qw / QX == round;  // wave-uniform
    __syncthreads();
    if (kh == 1 && mine) {
      xch[0] = mref;
      xch[64] = lt;
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) xch[64 * (2 + 16 * mt + r)] = acc[mt][r];
    }
    __syncthreads();
    if (kh == 0 && mine) {
      const float m1 = xch[0], l1 = xch[64];
      m = fmaxf(mref, m1);
      const float a0 = mref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mref - m) * c);
      const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m1 - m) * c);
      lt = lt * a0 + l1 * a1;
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mt][r] = acc[mt][r] * a0 + xch[64 * (2 + 16 * mt + r)] * a1;
    }
  }
  if (kh == 1) return;

  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qrow_e < a.Tq) {
    const int orow = a.orig_rows ? min(max(orow_raw, 0), a.Tqs - 1) : qrow_e;  // as out_row_q
    uint16_t *O = static_cast<uint16_t *>(a.out_o) + ((size_t)bh * a.Tqo + orow) * D;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mt + 8 * g + 4 * half_e;
        const uint2 val = make_uint2(pack_bf16x2(acc[mt][4 * g] * inv, acc[mt][4 * g + 1] * inv),
                                     pack_bf16x2(acc[mt][4 * g + 2] * inv, acc[mt][4 * g + 3] * inv));
        *reinterpret_cast<uint2 *>(O + d0) = val;
      }
    if (half_e == 0) a.out_lse[(size_t)bh * a.Tqo + orow] = lt > 0.f ? m * a.scale + logf(lt) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// fp32 forward: one thread per query row.
// ---------------------------------------------------------------------------
constexpr int kF32Chunk = 32;

template <int MODE, int D, int BS>
__global__ __launch_bounds__(BS) void k_fwd_f32(AttnArgs a) {
  __shared__ float sK[kF32Chunk][D];
  __shared__ float sV[kF32Chunk][D];
  __shared__ int sKidx[kF32Chunk];
  __shared__ int sKhash[kF32Chunk];
  const int bh = blockIdx.x / a.nq;
  const int qb = blockIdx.x % a.nq;
  if (varlen_head(a, bh, 4) && qb * BS >= a.Tq) return;  // past this ragged head's queries
  const int qrow = qb * BS + threadIdx.x;
  const bool qvalid = qrow < a.Tq;
  const float *Q = static_cast<const float *>(a.q) + (size_t)bh * a.Tq * D;
  const float *K = static_cast<const float *>(a.k) + (size_t)bh * a.Tk * D;
  const float *V = static_cast<const float *>(a.v) + (size_t)bh * a.Tk * D;
  float q[D], acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    q[i] = qvalid ? Q[(size_t)qrow * D + i] : 0.f;
    acc[i] = 0.f;
  }
  int my_idx = kIdxTailQ, my_hash = 0;
  if (qvalid) {
    my_idx = MODE == kDense ? qrow : a.q_idx[(size_t)bh * a.Tq + qrow];
    if (MODE == kHash) my_hash = a.q_hash[(size_t)bh * a.Tq + qrow];
  }
  LiveList rl = row_list<MODE, BS>(a, bh, qb);
  float m = -INFINITY, l = 0.f;
  for (int t = 0; t < rl.n; ++t) {
    int kb;
    bool free;
    tile_at<MODE, BS>(a, rl, t, qb, kb, free);
    if (kb >= a.nk) continue;
    const int kend = min((kb + 1) * BS, a.Tk);
    for (int k0 = kb * BS; k0 < kend; k0 += kF32Chunk) {
      const int kvalid = min(kF32Chunk, kend - k0);
      __syncthreads();
      for (int i = threadIdx.x; i < kF32Chunk * D; i += BS) {
        const int r = i / D, cc = i % D;
        sK[r][cc] = r < kvalid ? K[(size_t)(k0 + r) * D + cc] : 0.f;
        sV[r][cc] = r < kvalid ? V[(size_t)(k0 + r) * D + cc] : 0.f;
      }
      for (int r = threadIdx.x; r < kF32Chunk; r += BS) {
        sKidx[r] = r < kvalid ? (MODE == kDense ? k0 + r : a.k_idx[(size_t)bh * a.Tk + k0 + r]) : kIdxTailK;
        sKhash[r] = (MODE == kHash && r < kvalid) ? a.k_hash[(size_t)bh * a.Tk + k0 + r] : 0;
      }
      __syncthreads();
      float s[kF32Chunk];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kF32Chunk; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < D; ++i) dot = fmaf(q[i], sK[j][i], dot);
        const bool ok = j < kvalid && (free || (sKidx[j] <= my_idx && (MODE != kHash || sKhash[j] == my_hash)));
        s[j] = ok ? dot : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = expf((m - m_use) * a.scale);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] *= alpha;
#pragma unroll
      for (int j = 0; j < kF32Chunk; ++j) {
        const float p = expf((s[j] - m_use) * a.scale);
        l += p;
#pragma unroll
        for (int i = 0; i < D; ++i) acc[i] = fmaf(p, sV[j][i], acc[i]);
      }
      m = m_new;
    }
  }
  if (qvalid) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float *O = static_cast<float *>(a.out_o) + ((size_t)bh * a.Tq + qrow) * D;
#pragma unroll
    for (int i = 0; i < D; ++i) O[i] = acc[i] * inv;
    a.out_lse[(size_t)bh * a.Tq + qrow] = l > 0.f ? m * a.scale + logf(l) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
template <int MODE, int D, int BS>
static hipError_t run_fwd_bf16(const AttnArgs &a, hipStream_t s) {
  if constexpr (D == 128 && BS == 128 && MODE == kHash) {
    // 128-query blocks of the lists run as two 64-query groups: the 4-wave groups fit twice per CU
    // (the 8-wave group once), the same 8 waves per CU with half as many waiting at each barrier.
    // Each chunk is copied once per 64 queries instead of 128, which costs more than it saves on long
    // lists (dense and QK-sparse: equal or 2 % slower at 32k tokens, 21 % slower for dense causal at
    // 1M tokens, where a head's K and V outgrow the caches) and pays on the short lists of bucketed
    // attention (7-9 % faster at 64 and 256 buckets).
    const unsigned grid = (unsigned)(a.BH * ((a.Tq + 63) / 64));
    if (a.k_rows) hipLaunchKernelGGL((k_fwd_bf16_ks<MODE, D, 64, true, 128>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_fwd_bf16_ks<MODE, D, 64, false, 128>), dim3(grid), dim3(256), 0, s, a);
  } else {
    if (a.k_rows)
      hipLaunchKernelGGL((k_fwd_bf16_ks<MODE, D, BS, true>), dim3((unsigned)(a.BH * a.nq)), dim3(BS / 16 * 64), 0, s,
                         a);
    else
      hipLaunchKernelGGL((k_fwd_bf16_ks<MODE, D, BS, false>), dim3((unsigned)(a.BH * a.nq)), dim3(BS / 16 * 64), 0, s,
                         a);
  }
  return hipGetLastError();
}
template <int MODE, int D, int BS>
static hipError_t run_fwd_f32(const AttnArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((k_fwd_f32<MODE, D, BS>), dim3((unsigned)(a.BH * a.nq)), dim3(BS), 0, s, a);
  return hipGetLastError();
}

#define SCFA_DISPATCH(FN, a, mode, s)                                                       \
  do {                                                                                      \
    const int key = (mode) * 4 + ((a).d == 128 ? 2 : 0) + ((a).block == 128 ? 1 : 0);       \
    switch (key) {                                                                          \
      case 0: return FN<kDense, 64, 64>(a, s);                                              \
      case 1: return FN<kDense, 64, 128>(a, s);                                             \
      case 2: return FN<kDense, 128, 64>(a, s);                                             \
      case 3: return FN<kDense, 128, 128>(a, s);                                            \
      case 4: return FN<kQK, 64, 64>(a, s);                                                 \
      case 5: return FN<kQK, 64, 128>(a, s);                                                \
      case 6: return FN<kQK, 128, 64>(a, s);                                                \
      case 7: return FN<kQK, 128, 128>(a, s);                                               \
      case 8: return FN<kHash, 64, 64>(a, s);                                               \
      case 9: return FN<kHash, 64, 128>(a, s);                                              \
      case 10: return FN<kHash, 128, 64>(a, s);                                             \
      case 11: return FN<kHash, 128, 128>(a, s);                                            \
      default: return hipErrorInvalidValue;                                                 \
    }                                                                                       \
  } while (0)

hipError_t launch_attn_fwd_bf16(const AttnArgs &a, int mode, hipStream_t s) {
  if (a.BH == 0 || a.nq == 0) return hipSuccess;
  SCFA_DISPATCH(run_fwd_bf16, a, mode, s);
}

hipError_t launch_attn_fwd_f32(const AttnArgs &a, int mode, hipStream_t s) {
  if (a.BH == 0 || a.nq == 0) return hipSuccess;
  SCFA_DISPATCH(run_fwd_f32, a, mode, s);
}

}  // namespace scfa
