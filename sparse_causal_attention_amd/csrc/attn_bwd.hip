// SCFA backward: gradients of sum(O * dO) recomputing P from the saved
// log-sum-exp, over the same live tiles and element mask as the forward
// (deep-paper.org summary of arXiv 2306.01160, "SCFA solution": the tile
// rules apply to every kernel; the page reports training speedups, which
// need this pass, without describing it).
//
// Analytic gradients: D_i = dO_i . O_i, P = mask * exp(scale S - lse),
// dV = P^T dO, dP = dO V^T, dS = P * (dP - D), dQ = scale dS K,
// dK = scale dS^T Q.
//
// Two kernels, no atomics (results are deterministic):
//  * dQ kernel: one work group per query block, walking its row list (live
//    key blocks).  It also writes D for the dK/dV kernel.  Orientation as in
//    the forward (lanes own query columns): S^T = K Q^T, dP^T = V dO^T,
//    dQ^T += K^T dS^T.
//  * dK/dV kernel: one work group per key block, walking its column list
//    (live query blocks).  Lanes own key columns: S = Q K^T, dP = dO V^T,
//    dV^T += dO^T P, dK^T += Q^T dS.
//
// Stored-dS variant (bf16, pruned modes): a preprocess kernel writes D and
// lse * log2 e; the dK/dV kernel also stores every live tile's bf16 dS^T
// (key-major, the values its dK product uses) in that tile's slot; the dQ
// kernel is then a plain block-sparse product dQ^T += K^T dS^T over the row
// lists, with no exponent, mask or dP.  The recomputing dQ kernel stays as
// the fallback when the dS buffer is too small.
#include "scfa_device.hpp"
#include "scfa_internal.hpp"
#include "scfa_pipe.hpp"

namespace scfa {

template <int MODE, int BS>
__device__ __forceinline__ LiveList row_list_b(const AttnArgs &a, int bh, int qb) {
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

template <int MODE, int BS>
__device__ __forceinline__ void row_tile(const AttnArgs &a, LiveList &rl, int t, int qb, int &kb, bool &free) {
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

template <int MODE, int BS>
__device__ __forceinline__ LiveList col_list_b(const AttnArgs &a, int bh, int kb) {
  LiveList r{0, 0, nullptr, 0, 0, 0};
  if (a.no_prune) {
    r.n = a.nq;
  } else if (MODE == kDense) {
    // live(i, kb) iff min((i+1)*BS, Tq) - 1 >= kb*BS, i.e. i >= kb when kb*BS < Tq
    r.first = kb;
    r.n = kb * BS < a.Tq ? a.nq - kb : 0;
  } else {
    r.n = min(a.col_cnt[(size_t)bh * a.nk + kb], a.nq);
    r.p = a.col_list + ((size_t)bh * a.nk + kb) * a.nq;
    r.lim = a.nq;
    list_window(r, 0);
  }
  return r;
}

template <int MODE, int BS>
__device__ __forceinline__ void col_tile(const AttnArgs &a, LiveList &cl, int t, int kb, int &qb, bool &free) {
  if (a.no_prune) {
    qb = t;
    free = false;
  } else if (MODE == kDense) {
    qb = cl.first + t;
    free = min((kb + 1) * BS, a.Tk) - 1 <= qb * BS;
  } else {
    const int e = list_entry(cl, t);
    qb = e & 0x7fffffff;
    free = e < 0;
  }
  if (a.force_mask) free = false;
}

// ---------------------------------------------------------------------------
// Chunk iteration over a row list (dQ) or a column list (dK/dV).
// ---------------------------------------------------------------------------
struct Chunk {
  int t, ch, r0, nvalid;
  bool free;
  int slot;  // stored-dS slot of the chunk's tile (dQ kernel over stored dS), else -1
};

// `sl` (nullable): the entries' dS slots, read through a register window like the list.
template <int MODE, int BS, bool ROWS>
__device__ __forceinline__ bool next_chunk(const AttnArgs &a, LiveList &ls, int self, int t, int ch, Chunk &out,
                                           LiveList *sl = nullptr) {
  constexpr int NCH = BS / kChunk;
  const int n_other = ROWS ? a.nk : a.nq;
  const int T_other = ROWS ? a.Tk : a.Tq;
  for (; t < ls.n; ++t, ch = 0) {
    int ob;
    bool free;
    if (ROWS) row_tile<MODE, BS>(a, ls, t, self, ob, free);
    else col_tile<MODE, BS>(a, ls, t, self, ob, free);
    if (ob >= n_other || ch >= NCH) continue;
    const int r0 = ob * BS + ch * kChunk;
    if (r0 >= T_other) continue;
    out.t = t;
    out.ch = ch;
    out.r0 = r0;
    out.nvalid = min(kChunk, T_other - r0);
    out.free = free;
    out.slot = sl ? list_entry(*sl, t) : -1;
    return true;
  }
  return false;
}

template <int D>
struct KVBufB {
  MatChunk<D> k, v;
  int idx[kChunk];
  int hash[kChunk];
};

template <int D>
struct QGBuf {
  MatChunk<D> q, g;  // Q and dO rows
  float lse2[kChunk];
  float del[kChunk];
  int idx[kChunk];
  int hash[kChunk];
};

// ---------------------------------------------------------------------------
// bf16 dQ (+ D, lse*log2 e) kernel.  Lanes own query columns.
// ---------------------------------------------------------------------------
// KROWS: K and V chunk rows come through a.k_rows (indices loaded one chunk
// ahead); Q and dO rows come through a.q_rows when it is set.
template <int MODE, int D, int BS, bool KROWS>
__global__ __launch_bounds__(BS / 32 * 64) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1))) void k_bwd_dq_bf16(AttnArgs a) {
  constexpr int NW = BS / 32;
  __shared__ __attribute__((aligned(16))) KVBufB<D> sb[2];
  // As the stored-dS path's fallback, run only when the dS buffer was too small.
  if (a.dq_fallback && a.col_base[(size_t)a.BH * a.nk] <= a.ds_tiles) return;

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / a.nq;
  const int qb = wg % a.nq;
  if (varlen_head(a, bh, 2) && qb * BS >= a.Tq) return;  // past this ragged head's queries
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int qrow = qb * BS + 32 * w + col;
  const bool qvalid = qrow < a.Tq;
  const size_t qoff = (size_t)bh * a.Tq;  // view-indexed arrays (positions, buckets, rows)
  const size_t qoo = (size_t)bh * a.Tqo;  // the forward's outputs (o, lse) and dq
  const uint16_t *Q = static_cast<const uint16_t *>(a.q) + (size_t)bh * a.Tqs * D;
  const uint16_t *dO = static_cast<const uint16_t *>(a.dout) + (size_t)bh * a.Tqs * D;
  const uint16_t *O = static_cast<const uint16_t *>(a.o) + qoo * D;
  const uint16_t *K = static_cast<const uint16_t *>(a.k) + (size_t)bh * a.Tks * D;
  const uint16_t *V = static_cast<const uint16_t *>(a.v) + (size_t)bh * a.Tks * D;

  // Loads that depend only on this lane's own row go first: issued after the
  // list and chunk copies, a wait for them would also wait for those copies.
  int qsrc_raw = a.q_rows && qvalid ? a.q_rows[qoff + qrow] : qrow;  // clamped where used
  // lse (and O below) are read at the caller's row when outputs live there
  const int lrow = a.orig_rows && qvalid ? min(max(qsrc_raw, 0), a.Tqs - 1) : qrow;
  float lse_raw = qvalid ? a.lse[qoo + lrow] : 0.f;
  int my_idx = kIdxTailQ, my_hash = 0;
  if (qvalid) {
    my_idx = MODE == kDense ? qrow : a.q_idx[qoff + qrow];
    if (MODE == kHash) my_hash = a.q_hash[qoff + qrow];
  }
  LiveList rl = row_list_b<MODE, BS>(a, bh, qb);
  // Consumed here, where the list window's wait already covers these older loads;
  // first used after the chunk copies, their wait would also drain them.
  asm volatile("" : "+v"(qsrc_raw), "+v"(lse_raw));
  const DmaOffsets<D, NW> dmo = dma_offsets<D, NW>();
  const LaneOffsets<D> lo = lane_offsets<D>();
  const int32_t *krows = KROWS ? a.k_rows + (size_t)bh * a.Tk : nullptr;
  DmaRows<D, NW> drn;  // KROWS: source rows of the next chunk to copy
  auto issue = [&](KVBufB<D> &b, const Chunk &c) {
    if constexpr (KROWS) {
      dma_matrix_rows<D, NW>(b.k, K, a.Tks, drn);
      dma_matrix_rows<D, NW>(b.v, V, a.Tks, drn);
    } else {
      dma_matrix<D, NW>(b.k, K, c.r0, c.nvalid, dmo);
      dma_matrix<D, NW>(b.v, V, c.r0, c.nvalid, dmo);
    }
    if (MODE != kDense && !(c.free && c.nvalid == kChunk)) {
      if (w == 0) dma_vec(b.idx, a.k_idx + (size_t)bh * a.Tk, c.r0, c.nvalid);
      if (MODE == kHash && w == NW - 1) dma_vec(b.hash, a.k_hash + (size_t)bh * a.Tk, c.r0, c.nvalid);
    }
  };
  Chunk cur;
  bool have = next_chunk<MODE, BS, true>(a, rl, qb, 0, 0, cur);
  if (have) {
    if constexpr (KROWS) dma_rows_load<D, NW>(drn, krows, cur.r0, cur.nvalid);
    issue(sb[0], cur);
  }
  Chunk nxt;  // KROWS: looked up one chunk ahead, so its row indices can load early
  bool have_next = false;
  if constexpr (KROWS) {
    have_next = have && next_chunk<MODE, BS, true>(a, rl, qb, cur.t, cur.ch + 1, nxt);
    if (have_next) dma_rows_load<D, NW>(drn, krows, nxt.r0, nxt.nvalid);
  }

  const int qsrc = a.q_rows && qvalid ? min(max(qsrc_raw, 0), a.Tqs - 1) : qrow;
  bf16x8 qf[D / 16], dof[D / 16];
  float dsum = 0.f;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const size_t off = (size_t)(a.orig_rows ? qsrc : qrow) * D + 16 * kk + 8 * half;
    const size_t soff = (size_t)qsrc * D + 16 * kk + 8 * half;
    const uint4 z = make_uint4(0, 0, 0, 0);
    const uint4 uq = qvalid ? ld16(Q + soff) : z;
    const uint4 ud = qvalid ? ld16(dO + soff) : z;
    const uint4 uo = qvalid ? ld16(O + off) : z;
    qf[kk] = as_bf16x8(uq);
    dof[kk] = as_bf16x8(ud);
    const uint32_t dw[4] = {ud.x, ud.y, ud.z, ud.w};
    const uint32_t ow[4] = {uo.x, uo.y, uo.z, uo.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dsum = fmaf(bf16_bits_to_float(dw[e] & 0xffffu), bf16_bits_to_float(ow[e] & 0xffffu), dsum);
      dsum = fmaf(bf16_bits_to_float(dw[e] >> 16), bf16_bits_to_float(ow[e] >> 16), dsum);
    }
  }
  dsum = pair_sum(dsum);
  const float lse2 = qvalid ? lse_raw * kLog2e : INFINITY;
  if (qvalid && half == 0) {
    a.delta[qoff + qrow] = dsum;
    a.delta[a.delta_half + qoff + qrow] = lse2;
  }
  const float c = a.scale * kLog2e;
  f32x16 dqa[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[mt][r] = 0.f;

  int buf = 0;
  while (have) {
    Chunk nxt2;
    bool have_next2 = false;
    if constexpr (KROWS) have_next2 = have_next && next_chunk<MODE, BS, true>(a, rl, qb, nxt.t, nxt.ch + 1, nxt2);
    else have_next = next_chunk<MODE, BS, true>(a, rl, qb, cur.t, cur.ch + 1, nxt);
    wait_vmem();
    __syncthreads();
    if (have_next) issue(sb[buf ^ 1], nxt);
    if constexpr (KROWS)
      if (have_next2) dma_rows_load<D, NW>(drn, krows, nxt2.r0, nxt2.nvalid);
    const KVBufB<D> &b = sb[buf];

    // Fragments first, then four independent accumulator chains (S^T and
    // dP^T of both 32-key halves) interleaved with the k-step outermost.
    bf16x8 kfr[2][D / 16], vfr[2][D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        kfr[sub][kk] = frag_rows<D>(b.k, lo, sub, kk);
        vfr[sub][kk] = frag_rows<D>(b.v, lo, sub, kk);
      }
    f32x16 s[2], dp[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      s[sub] = mfma32(kfr[sub][0], qf[0], kZero16);
      dp[sub] = mfma32(vfr[sub][0], dof[0], kZero16);
    }
#pragma unroll
    for (int kk = 1; kk < D / 16; ++kk)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        s[sub] = mfma32(kfr[sub][kk], qf[kk], s[sub]);
        dp[sub] = mfma32(vfr[sub][kk], dof[kk], dp[sub]);
      }
    // K^T fragments of the dQ product, requested before the exponent work
    bf16x8 ktr[4][D / 32];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) ktr[t][mt] = frag_trans<D>(b.k, lo, mt, t);
    // P = exp(scale*S - lse); rows with no admissible key (lse = -inf) only
    // occur in masked tiles, where the select below discards them.
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[sub][r] = __builtin_amdgcn_exp2f(fmaf(s[sub][r], c, -lse2));
    if (cur.nvalid < kChunk)
      mask_rows<MODE, true>(s, b.idx, b.hash, cur.r0, cur.nvalid, my_idx, my_hash, half, 0.f);
    else if (!cur.free)
      mask_rows<MODE, false>(s, b.idx, b.hash, cur.r0, cur.nvalid, my_idx, my_hash, half, 0.f);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[sub][r] = s[sub][r] * (dp[sub][r] - dsum);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const bf16x8 db = as_bf16x8(c_regs_to_u4(s[sub], t2));
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) dqa[mt] = mfma32(ktr[2 * sub + t2][mt], db, dqa[mt]);
      }
    buf ^= 1;
    cur = nxt;
    have = have_next;
    if constexpr (KROWS) {
      nxt = nxt2;
      have_next = have_next2;
    }
  }

  // Store addresses recomputed from an opaque copy of the thread id (nothing
  // lane-derived stays live across the chunk loop).
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int qrow_e = qb * BS + 32 * (tid >> 6) + (tid & 31), half_e = (tid >> 5) & 1;
  if (qrow_e < a.Tq) {
    // The output row: lrow from the prologue (the caller's row with orig_rows)
    // where one more live register costs no spill, else loaded again here.
    const int orow = MODE != kDense ? lrow : out_row_q(a, bh, qrow_e);
    uint16_t *dQ = static_cast<uint16_t *>(a.dq) + (qoo + orow) * D;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mt + 8 * g + 4 * half_e;
        *reinterpret_cast<uint2 *>(dQ + d0) =
            make_uint2(pack_bf16x2(dqa[mt][4 * g] * a.scale, dqa[mt][4 * g + 1] * a.scale),
                       pack_bf16x2(dqa[mt][4 * g + 2] * a.scale, dqa[mt][4 * g + 3] * a.scale));
      }
  }
}

// ---------------------------------------------------------------------------
// bf16 dK / dV kernel.  Lanes own key columns.
// ---------------------------------------------------------------------------
// QROWS: Q and dO chunk rows come through a.q_rows (indices loaded one chunk
// ahead); K and V rows come through a.k_rows when it is set.
// STORE: also write each tile's bf16 dS^T into its slot (col_base[bh*nk + kb]
// + list position), unless the buffer is too small for all tiles.  A tile is
// stored as 16-query groups, [BS/16][BS keys][16 queries], so each store
// instruction writes a contiguous kilobyte.
template <int MODE, int D, int BS, bool QROWS, bool STORE>
__global__ __launch_bounds__(BS / 32 * 64) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1))) void k_bwd_dkdv_bf16(AttnArgs a) {
  constexpr int NW = BS / 32;
  __shared__ __attribute__((aligned(16))) QGBuf<D> sb[2];

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / a.nk;
  const int kb = wg % a.nk;
  if (varlen_head(a, bh, 2) && kb * BS >= a.Tk) return;  // past this ragged head's keys
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int krow = kb * BS + 32 * w + col;
  const bool kvalid_row = krow < a.Tk;
  const size_t koff = (size_t)bh * a.Tk;  // view-indexed arrays (positions, buckets, rows)
  const size_t qoff = (size_t)bh * a.Tq;
  const uint16_t *Q = static_cast<const uint16_t *>(a.q) + (size_t)bh * a.Tqs * D;
  const uint16_t *dO = static_cast<const uint16_t *>(a.dout) + (size_t)bh * a.Tqs * D;
  const uint16_t *K = static_cast<const uint16_t *>(a.k) + (size_t)bh * a.Tks * D;
  const uint16_t *V = static_cast<const uint16_t *>(a.v) + (size_t)bh * a.Tks * D;
  const float *lse2g = a.delta + a.delta_half + qoff;
  const float *delg = a.delta + qoff;

  // Loads that depend only on this lane's own row go first: issued after the
  // list and chunk copies, a wait for them would also wait for those copies.
  int ksrc_raw = a.k_rows && kvalid_row ? a.k_rows[koff + krow] : krow;  // clamped where used
  int my_idx = kIdxTailK, my_hash = 0;
  if (kvalid_row) {
    my_idx = MODE == kDense ? krow : a.k_idx[koff + krow];
    if (MODE == kHash) my_hash = a.k_hash[koff + krow];
  }
  LiveList cl = col_list_b<MODE, BS>(a, bh, kb);
  // STORE: this key block's first dS slot (its tiles take consecutive slots in list order)
  const int slot0 = STORE ? a.col_base[(size_t)bh * a.nk + kb] : 0;
  const bool store = STORE && a.col_base[(size_t)a.BH * a.nk] <= a.ds_tiles;
  // Consumed here, where the list window's wait already covers this older load;
  // first used after the chunk copies, its wait would also drain them.
  asm volatile("" : "+v"(ksrc_raw));
  const DmaOffsets<D, NW> dmo = dma_offsets<D, NW>();
  const LaneOffsets<D> lo = lane_offsets<D>();
  const int32_t *qrows = QROWS ? a.q_rows + qoff : nullptr;
  // STORE on a key block with rows past Tk: every chunk is masked, so those rows
  // (position kIdxTailK, after every query) get P = 0 and store dS = 0.
  const bool mask_all = STORE && (kb + 1) * BS > a.Tk;
  DmaRows<D, NW> drn;  // QROWS: source rows of the next chunk to copy
  auto issue = [&](QGBuf<D> &b, const Chunk &c) {
    if constexpr (QROWS) {
      dma_matrix_rows<D, NW>(b.q, Q, a.Tqs, drn);
      dma_matrix_rows<D, NW>(b.g, dO, a.Tqs, drn);
    } else {
      dma_matrix<D, NW>(b.q, Q, c.r0, c.nvalid, dmo);
      dma_matrix<D, NW>(b.g, dO, c.r0, c.nvalid, dmo);
    }
    if (w == 0) dma_vec(b.lse2, lse2g, c.r0, c.nvalid);
    if (w == NW - 1) dma_vec(b.del, delg, c.r0, c.nvalid);
    if (MODE != kDense && (mask_all || !(c.free && c.nvalid == kChunk))) {
      if (w == 0) dma_vec(b.idx, a.q_idx + qoff, c.r0, c.nvalid);
      if (MODE == kHash && w == NW - 1) dma_vec(b.hash, a.q_hash + qoff, c.r0, c.nvalid);
    }
  };
  Chunk cur;
  bool have = next_chunk<MODE, BS, false>(a, cl, kb, 0, 0, cur);
  if (have) {
    if constexpr (QROWS) dma_rows_load<D, NW>(drn, qrows, cur.r0, cur.nvalid);
    issue(sb[0], cur);
  }
  Chunk nxt;  // QROWS: looked up one chunk ahead, so its row indices can load early
  bool have_next = false;
  if constexpr (QROWS) {
    have_next = have && next_chunk<MODE, BS, false>(a, cl, kb, cur.t, cur.ch + 1, nxt);
    if (have_next) dma_rows_load<D, NW>(drn, qrows, nxt.r0, nxt.nvalid);
  }

  const int ksrc = a.k_rows && kvalid_row ? min(max(ksrc_raw, 0), a.Tks - 1) : krow;
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const size_t off = (size_t)ksrc * D + 16 * kk + 8 * half;
    kf[kk] = as_bf16x8(kvalid_row ? ld16(K + off) : make_uint4(0, 0, 0, 0));
    vf[kk] = as_bf16x8(kvalid_row ? ld16(V + off) : make_uint4(0, 0, 0, 0));
  }
  const float c = a.scale * kLog2e;
  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dka[mt][r] = 0.f;
      dva[mt][r] = 0.f;
    }

  // STORE: the dS^T of a chunk's second 32-query half is held in registers and
  // stored after the next chunk's top-of-loop wait.  Stores count in the same
  // counter as the chunk copies, so a store issued at the end of a chunk would
  // be waited for right away by that wait; issued after it, the store has a
  // whole chunk to complete.
  uint4 held[2] = {};
  size_t held_off = 0;  // element offset of the held half's 16-query block in ds (lane part excluded)
  bool held_valid = false;
  const size_t lane_ds = (size_t)(32 * w + col) * 16 + 8 * half;  // this lane's key row and query octet
  auto store_held = [&](size_t lane_off) {
    uint16_t *p = static_cast<uint16_t *>(a.ds) + held_off + lane_off;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) *reinterpret_cast<uint4 *>(p + (size_t)t2 * BS * 16) = held[t2];
  };

  int buf = 0;
  while (have) {
    Chunk nxt2;
    bool have_next2 = false;
    if constexpr (QROWS) have_next2 = have_next && next_chunk<MODE, BS, false>(a, cl, kb, nxt.t, nxt.ch + 1, nxt2);
    else have_next = next_chunk<MODE, BS, false>(a, cl, kb, cur.t, cur.ch + 1, nxt);
    wait_vmem();
    __syncthreads();
    if (have_next) issue(sb[buf ^ 1], nxt);
    if constexpr (QROWS)
      if (have_next2) dma_rows_load<D, NW>(drn, qrows, nxt2.r0, nxt2.nvalid);
    if constexpr (STORE) {
      if (held_valid) store_held(lane_ds);
      held_valid = false;
    }
    const QGBuf<D> &b = sb[buf];
    // Key rows past Tk only pollute their own (never stored) columns, so a
    // mask-free tile needs masking only for query rows past Tq.
    // The chunk is processed as two halves of 32 query rows; each half is
    // S, dP (4 independent chains) -> P, dS -> dV^T, dK^T, so the second
    // half's products can overlap the first half's exponent and mask work.
    const bool tail = cur.nvalid < kChunk, masked = tail || !cur.free || mask_all;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      bf16x8 qfr[D / 16], gfr[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        qfr[kk] = frag_rows<D>(b.q, lo, sub, kk);
        gfr[kk] = frag_rows<D>(b.g, lo, sub, kk);
      }
      f32x16 s1[1], dp1[1];
      s1[0] = mfma32(qfr[0], kf[0], kZero16);
      dp1[0] = mfma32(gfr[0], vf[0], kZero16);
#pragma unroll
      for (int kk = 1; kk < D / 16; ++kk) {
        s1[0] = mfma32(qfr[kk], kf[kk], s1[0]);
        dp1[0] = mfma32(gfr[kk], vf[kk], dp1[0]);
      }
      bf16x8 gtr[2][D / 32], qtr[2][D / 32];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
          gtr[t2][mt] = frag_trans<D>(b.g, lo, mt, 2 * sub + t2);
          qtr[t2][mt] = frag_trans<D>(b.q, lo, mt, 2 * sub + t2);
        }
      // P = exp(scale*S - lse) per query row (lse * log2 e staged in LDS).
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 l4 = *reinterpret_cast<const float4 *>(b.lse2 + 32 * sub + 8 * g + 4 * half);
        s1[0][4 * g + 0] = __builtin_amdgcn_exp2f(fmaf(s1[0][4 * g + 0], c, -l4.x));
        s1[0][4 * g + 1] = __builtin_amdgcn_exp2f(fmaf(s1[0][4 * g + 1], c, -l4.y));
        s1[0][4 * g + 2] = __builtin_amdgcn_exp2f(fmaf(s1[0][4 * g + 2], c, -l4.z));
        s1[0][4 * g + 3] = __builtin_amdgcn_exp2f(fmaf(s1[0][4 * g + 3], c, -l4.w));
      }
      if (tail)
        mask_half<MODE, true>(s1[0], b.idx, b.hash, 32 * sub, cur.r0, cur.nvalid, my_idx, my_hash, half, 0.f);
      else if (masked)
        mask_half<MODE, false>(s1[0], b.idx, b.hash, 32 * sub, cur.r0, cur.nvalid, my_idx, my_hash, half, 0.f);
      // dS = P * (dP - D)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 d4 = *reinterpret_cast<const float4 *>(b.del + 32 * sub + 8 * g + 4 * half);
        dp1[0][4 * g + 0] = s1[0][4 * g + 0] * (dp1[0][4 * g + 0] - d4.x);
        dp1[0][4 * g + 1] = s1[0][4 * g + 1] * (dp1[0][4 * g + 1] - d4.y);
        dp1[0][4 * g + 2] = s1[0][4 * g + 2] * (dp1[0][4 * g + 2] - d4.z);
        dp1[0][4 * g + 3] = s1[0][4 * g + 3] * (dp1[0][4 * g + 3] - d4.w);
      }
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const bf16x8 pb = as_bf16x8(c_regs_to_u4(s1[0], t2));
        const uint4 du = c_regs_to_u4(dp1[0], t2);
        const bf16x8 db = as_bf16x8(du);
        uint4 dsw = {};  // STORE: 8 consecutive queries of this lane's key (see below)
        if constexpr (STORE) {
          // Lane halves hold the query quads {0-3, 8-11} (half 0) and {4-7, 12-15} (half 1) of this
          // 16-query group (x, y: first quad; z, w: second).  Half 0 sends its second quad and takes
          // the partner's first; half 1 the reverse: queries 0-7 end in half 0, 8-15 in half 1.
          const uint32_t s0 = half ? du.x : du.z, s1 = half ? du.y : du.w;
          const uint32_t r0 = __shfl_xor(s0, 32, 64), r1 = __shfl_xor(s1, 32, 64);
          dsw = half ? make_uint4(r0, r1, du.z, du.w) : make_uint4(du.x, du.y, r0, r1);
        }
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
          dva[mt] = mfma32(gtr[t2][mt], pb, dva[mt]);
          dka[mt] = mfma32(qtr[t2][mt], db, dka[mt]);
        }
        if constexpr (STORE) {
          // Tile layout: 16-query groups [BS/16][BS keys][16 queries]; this (ch, sub, t2) is group
          // 4 ch + 2 sub + t2, and one wave's store covers 32 keys x 32 bytes, contiguous.
          // (a slot outside the buffer, from inconsistent caller slots, is not stored)
          const long long slot = (long long)slot0 + cur.t;
          if (store && slot >= 0 && slot < a.ds_tiles) {
            const size_t off = (size_t)slot * BS * BS + (size_t)(4 * cur.ch + 2 * sub) * BS * 16;
            if (sub == 0) {
              *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.ds) + off + (size_t)t2 * BS * 16 + lane_ds) = dsw;
            } else {
              held[t2] = dsw;
              held_off = off;
              held_valid = true;
            }
          }
        }
      }
    }
    buf ^= 1;
    cur = nxt;
    have = have_next;
    if constexpr (QROWS) {
      nxt = nxt2;
      have_next = have_next2;
    }
  }
  if constexpr (STORE) {
    if (held_valid) {
      int tid = threadIdx.x;  // lane offset recomputed: nothing lane-derived stays live past the loop
      asm volatile("" : "+v"(tid));
      store_held((size_t)(32 * (tid >> 6) + (tid & 31)) * 16 + 8 * ((tid >> 5) & 1));  // as lane_ds
    }
  }

  if (kvalid_row) {
    // The store addresses are recomputed here from an opaque copy of the thread
    // id, so no address stays live across the chunk loop.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int krow_e = kb * BS + 32 * (tid >> 6) + (tid & 31);
    const int half_e = (tid >> 5) & 1;
    // With orig_rows the output row is the row the K and V loads read (the
    // clamped k_rows entry, kept from the prologue where one more live
    // register costs no spill, else loaded again here).
    const size_t orow = STORE ? (size_t)out_row_k(a, bh, krow_e) : a.orig_rows ? (size_t)ksrc : (size_t)krow_e;
    uint16_t *dK = static_cast<uint16_t *>(a.dk) + ((size_t)bh * a.Tko + orow) * D;
    uint16_t *dV = static_cast<uint16_t *>(a.dv) + ((size_t)bh * a.Tko + orow) * D;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mt + 8 * g + 4 * half_e;
        *reinterpret_cast<uint2 *>(dK + d0) =
            make_uint2(pack_bf16x2(dka[mt][4 * g] * a.scale, dka[mt][4 * g + 1] * a.scale),
                       pack_bf16x2(dka[mt][4 * g + 2] * a.scale, dka[mt][4 * g + 3] * a.scale));
        *reinterpret_cast<uint2 *>(dV + d0) = make_uint2(pack_bf16x2(dva[mt][4 * g], dva[mt][4 * g + 1]),
                                                         pack_bf16x2(dva[mt][4 * g + 2], dva[mt][4 * g + 3]));
      }
  }
}

// ---------------------------------------------------------------------------
// Backward preprocess (stored-dS path): D = rowsum(dO * O) and lse * log2 e,
// summed exactly as the recomputing dQ kernel sums them (each 64-lane half of
// a row's 16-column groups sequentially with fused multiply-adds, then the
// two halves added), so both paths see the same D.  Two lanes per row.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_bwd_prep(AttnArgs a) {
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = g >> 1;  // over BH * Tq
  const int half = (int)(g & 1);
  const bool valid = row < (long long)a.BH * a.Tq;
  float dsum = 0.f;
  float lse = 0.f;
  if (valid) {
    const long long bh = row / a.Tq;
    const int i = (int)(row - bh * a.Tq);
    const int src = a.q_rows ? min(max(a.q_rows[row], 0), a.Tqs - 1) : i;
    const uint16_t *dO = static_cast<const uint16_t *>(a.dout) + ((size_t)bh * a.Tqs + src) * D;
    const size_t orow = a.orig_rows ? (size_t)bh * a.Tqo + src : (size_t)row;  // o and lse at the caller's rows
    const uint16_t *O = static_cast<const uint16_t *>(a.o) + orow * D;
    lse = a.lse[orow];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const uint4 ud = ld16(dO + 16 * kk + 8 * half), uo = ld16(O + 16 * kk + 8 * half);
      const uint32_t dw[4] = {ud.x, ud.y, ud.z, ud.w};
      const uint32_t ow[4] = {uo.x, uo.y, uo.z, uo.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dsum = fmaf(bf16_bits_to_float(dw[e] & 0xffffu), bf16_bits_to_float(ow[e] & 0xffffu), dsum);
        dsum = fmaf(bf16_bits_to_float(dw[e] >> 16), bf16_bits_to_float(ow[e] >> 16), dsum);
      }
    }
  }
  const float other = __shfl_xor(dsum, 1, 64);
  if (valid && half == 0) {
    a.delta[row] = dsum + other;
    a.delta[a.delta_half + row] = lse * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dQ from stored dS: one work group per query block walking its row list;
// entry t's tile is in slot row_slot[t] (read through a register window like
// the list).  2*BS/32 waves: wave w owns queries 32*(w % QW)..+31 (QW = BS/32)
// and half of the head dimension (d-tiles (w / QW)*D/64 ..), so twice the
// waves share each staged chunk.  Each 64-key chunk stages the K rows (through
// a.k_rows when KROWS) and the tile's dS^T rows [64 keys][BS queries] in LDS;
// both operands of dQ^T += K^T dS^T are transposed reads over the same key
// rows.
// ---------------------------------------------------------------------------
template <int D, int BS>
struct DsBuf {
  MatChunk<D> k;
  MatChunk<BS> ds;
};

// DMA source offsets that gather one 64-key chunk of a stored tile (16-query
// groups [BS/16][BS keys][16 queries], offsets relative to the chunk's first
// key row) into the row-major swizzled MatChunk<BS> layout: LDS piece s holds
// logical piece lp = (s % CPR) ^ swz<BS>(r) (queries 8 lp..) of chunk row r = s / CPR.
template <int BS, int NW>
__device__ __forceinline__ DmaOffsets<BS, NW> dma_offsets_ds() {
  using O = DmaOffsets<BS, NW>;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  O o;
#pragma unroll
  for (int k = 0; k < O::PER_WAVE; ++k) {
    const int s = (k * NW + w) * 64 + lane;
    const int r = s / O::CPR, lp = (s % O::CPR) ^ swz<BS>(r);
    o.off[k] = (lp >> 1) * BS * 16 + r * 16 + (lp & 1) * 8;
  }
  return o;
}

template <int D, int BS, bool KROWS>
__global__ __launch_bounds__(BS / 16 * 64) void k_bwd_dq_ds_bf16(AttnArgs a) {
  constexpr int QW = BS / 32;
  constexpr int NW = 2 * QW;
  constexpr int MTW = D / 64;  // d-tiles of 32 per wave
  __shared__ __attribute__((aligned(16))) DsBuf<D, BS> sb[2];
  if (a.col_base[(size_t)a.BH * a.nk] > a.ds_tiles) return;  // tiles not stored: the fallback computes dQ

  // Query blocks in reverse order: the dK/dV kernel wrote the tiles in roughly ascending block order, so
  // the most recently written (still cached) tiles are read first.
  const int wg = (int)gridDim.x - 1 - xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / a.nq;
  const int qb = wg % a.nq;
  const int w = threadIdx.x >> 6;
  const int qw = w % QW, mh = w / QW;
  const uint16_t *K = static_cast<const uint16_t *>(a.k) + (size_t)bh * a.Tks * D;
  const uint16_t *DS = static_cast<const uint16_t *>(a.ds);
  const size_t row = (size_t)bh * a.nq + qb;
  LiveList rl{min(a.row_cnt[row], a.nk), 0, a.row_list + row * a.nk, a.nk, 0, 0};
  LiveList sl{rl.n, 0, a.row_slot + row * a.nk, a.nk, 0, 0};
  list_window2(rl, sl, 0);
  const DmaOffsets<D, NW> dmk = dma_offsets<D, NW>();
  const DmaOffsets<BS, NW> dms = dma_offsets_ds<BS, NW>();
  int k_off[MTW], k_off2[MTW];
#pragma unroll
  for (int i = 0; i < MTW; ++i) {
    k_off[i] = trans_offset<D>(mh * MTW + i, 0);
    k_off2[i] = trans_offset<D>(mh * MTW + i, 1);
  }
  const int ds_off = trans_offset<BS>(qw, 0), ds_off2 = trans_offset<BS>(qw, 1);  // this wave's 32 query columns
  const int32_t *krows = KROWS ? a.k_rows + (size_t)bh * a.Tk : nullptr;
  DmaRows<D, NW> drn;  // KROWS: source rows of the next chunk to copy
  auto issue = [&](DsBuf<D, BS> &b, const Chunk &c) {
    if constexpr (KROWS) dma_matrix_rows<D, NW>(b.k, K, a.Tks, drn);
    else dma_matrix<D, NW>(b.k, K, c.r0, c.nvalid, dmk);
    // (an entry without a slot, which lists from the builder never have, reads tile 0)
    const size_t slot = (size_t)max(min(c.slot, (int)min(a.ds_tiles - 1, (long long)INT32_MAX)), 0);
    dma_matrix<BS, NW>(b.ds, DS + slot * BS * BS + (size_t)c.ch * kChunk * 16, 0, kChunk, dms);
  };
  Chunk cur;
  bool have = next_chunk<kQK, BS, true>(a, rl, qb, 0, 0, cur, &sl);
  if (have) {
    if constexpr (KROWS) dma_rows_load<D, NW>(drn, krows, cur.r0, cur.nvalid);
    issue(sb[0], cur);
  }
  Chunk nxt;
  bool have_next = false;
  if constexpr (KROWS) {
    have_next = have && next_chunk<kQK, BS, true>(a, rl, qb, cur.t, cur.ch + 1, nxt, &sl);
    if (have_next) dma_rows_load<D, NW>(drn, krows, nxt.r0, nxt.nvalid);
  }
  f32x16 dqa[MTW];
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[i][r] = 0.f;

  int buf = 0;
  while (have) {
    Chunk nxt2;
    bool have_next2 = false;
    if constexpr (KROWS)
      have_next2 = have_next && next_chunk<kQK, BS, true>(a, rl, qb, nxt.t, nxt.ch + 1, nxt2, &sl);
    else have_next = next_chunk<kQK, BS, true>(a, rl, qb, cur.t, cur.ch + 1, nxt, &sl);
    wait_vmem();
    __syncthreads();
    if (have_next) issue(sb[buf ^ 1], nxt);
    if constexpr (KROWS)
      if (have_next2) dma_rows_load<D, NW>(drn, krows, nxt2.r0, nxt2.nvalid);
    const DsBuf<D, BS> &b = sb[buf];
    bf16x8 ktr[4][MTW], dsb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      dsb[t] = frag_trans_at<BS>(b.ds, ds_off, ds_off2, t);
#pragma unroll
      for (int i = 0; i < MTW; ++i) ktr[t][i] = frag_trans_at<D>(b.k, k_off[i], k_off2[i], t);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < MTW; ++i) dqa[i] = mfma32(ktr[t][i], dsb[t], dqa[i]);
    buf ^= 1;
    cur = nxt;
    have = have_next;
    if constexpr (KROWS) {
      nxt = nxt2;
      have_next = have_next2;
    }
  }

  int tid = threadIdx.x;  // store addresses recomputed: nothing lane-derived stays live across the loop
  asm volatile("" : "+v"(tid));
  const int qrow_e = qb * BS + 32 * ((tid >> 6) % QW) + (tid & 31), half_e = (tid >> 5) & 1;
  if (qrow_e < a.Tq) {
    uint16_t *dQ = static_cast<uint16_t *>(a.dq) + ((size_t)bh * a.Tqo + out_row_q(a, bh, qrow_e)) * D;
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * (mh * MTW + i) + 8 * g + 4 * half_e;
        *reinterpret_cast<uint2 *>(dQ + d0) =
            make_uint2(pack_bf16x2(dqa[i][4 * g] * a.scale, dqa[i][4 * g + 1] * a.scale),
                       pack_bf16x2(dqa[i][4 * g + 2] * a.scale, dqa[i][4 * g + 3] * a.scale));
      }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernels: one thread per query row (dQ, D) / per key row (dK, dV).
// ---------------------------------------------------------------------------
constexpr int kF32Chunk = 32;

template <int MODE, int D, int BS>
__global__ __launch_bounds__(BS) void k_bwd_dq_f32(AttnArgs a) {
  __shared__ float sK[kF32Chunk][D];
  __shared__ float sV[kF32Chunk][D];
  __shared__ int sKidx[kF32Chunk];
  __shared__ int sKhash[kF32Chunk];
  const int bh = blockIdx.x / a.nq;
  const int qb = blockIdx.x % a.nq;
  if (varlen_head(a, bh, 4) && qb * BS >= a.Tq) return;  // past this ragged head's queries
  const int qrow = qb * BS + threadIdx.x;
  const bool qvalid = qrow < a.Tq;
  const size_t qoff = (size_t)bh * a.Tq;
  const float *Q = static_cast<const float *>(a.q) + qoff * D;
  const float *dO = static_cast<const float *>(a.dout) + qoff * D;
  const float *O = static_cast<const float *>(a.o) + qoff * D;
  const float *K = static_cast<const float *>(a.k) + (size_t)bh * a.Tk * D;
  const float *V = static_cast<const float *>(a.v) + (size_t)bh * a.Tk * D;
  float q[D], g[D], dq[D];
  float dsum = 0.f;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    q[i] = qvalid ? Q[(size_t)qrow * D + i] : 0.f;
    g[i] = qvalid ? dO[(size_t)qrow * D + i] : 0.f;
    dsum = fmaf(g[i], qvalid ? O[(size_t)qrow * D + i] : 0.f, dsum);
    dq[i] = 0.f;
  }
  if (qvalid) a.delta[qoff + qrow] = dsum;
  const float lse = qvalid ? a.lse[qoff + qrow] : INFINITY;
  int my_idx = kIdxTailQ, my_hash = 0;
  if (qvalid) {
    my_idx = MODE == kDense ? qrow : a.q_idx[qoff + qrow];
    if (MODE == kHash) my_hash = a.q_hash[qoff + qrow];
  }
  LiveList rl = row_list_b<MODE, BS>(a, bh, qb);
  for (int t = 0; t < rl.n; ++t) {
    int kb;
    bool free;
    row_tile<MODE, BS>(a, rl, t, qb, kb, free);
    if (kb >= a.nk) continue;  // entries outside the sequence are skipped
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
      for (int j = 0; j < kF32Chunk; ++j) {
        const bool ok = j < kvalid && (free || (sKidx[j] <= my_idx && (MODE != kHash || sKhash[j] == my_hash)));
        if (!ok) continue;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int i = 0; i < D; ++i) {
          s = fmaf(q[i], sK[j][i], s);
          dp = fmaf(g[i], sV[j][i], dp);
        }
        const float p = expf(s * a.scale - lse);
        const float ds = p * (dp - dsum);
#pragma unroll
        for (int i = 0; i < D; ++i) dq[i] = fmaf(ds, sK[j][i], dq[i]);
      }
    }
  }
  if (qvalid) {
    float *dQ = static_cast<float *>(a.dq) + (qoff + qrow) * D;
#pragma unroll
    for (int i = 0; i < D; ++i) dQ[i] = dq[i] * a.scale;
  }
}

template <int MODE, int D, int BS>
__global__ __launch_bounds__(BS) void k_bwd_dkdv_f32(AttnArgs a) {
  __shared__ float sQ[kF32Chunk][D];
  __shared__ float sG[kF32Chunk][D];
  __shared__ float sLse[kF32Chunk];
  __shared__ float sDel[kF32Chunk];
  __shared__ int sQidx[kF32Chunk];
  __shared__ int sQhash[kF32Chunk];
  const int bh = blockIdx.x / a.nk;
  const int kb = blockIdx.x % a.nk;
  if (varlen_head(a, bh, 4) && kb * BS >= a.Tk) return;  // past this ragged head's keys
  const int krow = kb * BS + threadIdx.x;
  const bool kvalid_row = krow < a.Tk;
  const size_t koff = (size_t)bh * a.Tk;
  const size_t qoff = (size_t)bh * a.Tq;
  const float *Q = static_cast<const float *>(a.q) + qoff * D;
  const float *dO = static_cast<const float *>(a.dout) + qoff * D;
  const float *K = static_cast<const float *>(a.k) + koff * D;
  const float *V = static_cast<const float *>(a.v) + koff * D;
  float kr[D], vr[D], dk[D], dv[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    kr[i] = kvalid_row ? K[(size_t)krow * D + i] : 0.f;
    vr[i] = kvalid_row ? V[(size_t)krow * D + i] : 0.f;
    dk[i] = 0.f;
    dv[i] = 0.f;
  }
  int my_idx = kIdxTailK, my_hash = 0;
  if (kvalid_row) {
    my_idx = MODE == kDense ? krow : a.k_idx[koff + krow];
    if (MODE == kHash) my_hash = a.k_hash[koff + krow];
  }
  LiveList cl = col_list_b<MODE, BS>(a, bh, kb);
  for (int t = 0; t < cl.n; ++t) {
    int qb;
    bool free;
    col_tile<MODE, BS>(a, cl, t, kb, qb, free);
    if (qb >= a.nq) continue;
    const int qend = min((qb + 1) * BS, a.Tq);
    for (int q0 = qb * BS; q0 < qend; q0 += kF32Chunk) {
      const int qv = min(kF32Chunk, qend - q0);
      __syncthreads();
      for (int i = threadIdx.x; i < kF32Chunk * D; i += BS) {
        const int r = i / D, cc = i % D;
        sQ[r][cc] = r < qv ? Q[(size_t)(q0 + r) * D + cc] : 0.f;
        sG[r][cc] = r < qv ? dO[(size_t)(q0 + r) * D + cc] : 0.f;
      }
      for (int r = threadIdx.x; r < kF32Chunk; r += BS) {
        const bool ok = r < qv;
        sLse[r] = ok ? a.lse[qoff + q0 + r] : INFINITY;
        sDel[r] = ok ? a.delta[qoff + q0 + r] : 0.f;
        sQidx[r] = ok ? (MODE == kDense ? q0 + r : a.q_idx[qoff + q0 + r]) : kIdxTailQ;
        sQhash[r] = (MODE == kHash && ok) ? a.q_hash[qoff + q0 + r] : 0;
      }
      __syncthreads();
      for (int i2 = 0; i2 < kF32Chunk; ++i2) {
        const bool ok = i2 < qv && (free || (my_idx <= sQidx[i2] && (MODE != kHash || sQhash[i2] == my_hash)));
        if (!ok) continue;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int i = 0; i < D; ++i) {
          s = fmaf(sQ[i2][i], kr[i], s);
          dp = fmaf(sG[i2][i], vr[i], dp);
        }
        const float p = expf(s * a.scale - sLse[i2]);
        const float ds = p * (dp - sDel[i2]);
#pragma unroll
        for (int i = 0; i < D; ++i) {
          dv[i] = fmaf(p, sG[i2][i], dv[i]);
          dk[i] = fmaf(ds, sQ[i2][i], dk[i]);
        }
      }
    }
  }
  if (kvalid_row) {
    float *dK = static_cast<float *>(a.dk) + (koff + krow) * D;
    float *dV = static_cast<float *>(a.dv) + (koff + krow) * D;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      dK[i] = dk[i] * a.scale;
      dV[i] = dv[i];
    }
  }
}

// ---------------------------------------------------------------------------
// part: bit 0 = dQ (+ D) kernel, bit 1 = dK/dV kernel (which reads D).
template <int MODE, int D, int BS>
static hipError_t run_bwd_bf16(const AttnArgs &a, int part, hipStream_t s) {
  if ((part & 1) && a.nq > 0) {
    if (a.k_rows)
      hipLaunchKernelGGL((k_bwd_dq_bf16<MODE, D, BS, true>), dim3((unsigned)(a.BH * a.nq)), dim3(BS / 32 * 64), 0, s, a);
    else
      hipLaunchKernelGGL((k_bwd_dq_bf16<MODE, D, BS, false>), dim3((unsigned)(a.BH * a.nq)), dim3(BS / 32 * 64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((part & 2) && a.nk > 0) {
    if (a.q_rows)
      hipLaunchKernelGGL((k_bwd_dkdv_bf16<MODE, D, BS, true, false>), dim3((unsigned)(a.BH * a.nk)), dim3(BS / 32 * 64), 0,
                         s, a);
    else
      hipLaunchKernelGGL((k_bwd_dkdv_bf16<MODE, D, BS, false, false>), dim3((unsigned)(a.BH * a.nk)), dim3(BS / 32 * 64),
                         0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int MODE, int D, int BS>
static hipError_t run_bwd_f32(const AttnArgs &a, int part, hipStream_t s) {
  if ((part & 1) && a.nq > 0) {
    hipLaunchKernelGGL((k_bwd_dq_f32<MODE, D, BS>), dim3((unsigned)(a.BH * a.nq)), dim3(BS), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((part & 2) && a.nk > 0) {
    hipLaunchKernelGGL((k_bwd_dkdv_f32<MODE, D, BS>), dim3((unsigned)(a.BH * a.nk)), dim3(BS), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

// Stored-dS backward.  part 2: dK/dV, storing the dS tiles; part 1: dQ from
// them, then the recomputing dQ kernel as the guarded fallback (it exits at
// once unless the buffer was too small).
template <int MODE, int D, int BS>
static hipError_t run_bwd_ds_bf16(const AttnArgs &a, int part, hipStream_t s) {
  if ((part & 2) && a.nk > 0) {
    if (a.q_rows)
      hipLaunchKernelGGL((k_bwd_dkdv_bf16<MODE, D, BS, true, true>), dim3((unsigned)(a.BH * a.nk)), dim3(BS / 32 * 64), 0,
                         s, a);
    else
      hipLaunchKernelGGL((k_bwd_dkdv_bf16<MODE, D, BS, false, true>), dim3((unsigned)(a.BH * a.nk)), dim3(BS / 32 * 64),
                         0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((part & 1) && a.nq > 0) {
    if (a.k_rows)
      hipLaunchKernelGGL((k_bwd_dq_ds_bf16<D, BS, true>), dim3((unsigned)(a.BH * a.nq)), dim3(BS / 16 * 64), 0, s, a);
    else
      hipLaunchKernelGGL((k_bwd_dq_ds_bf16<D, BS, false>), dim3((unsigned)(a.BH * a.nq)), dim3(BS / 16 * 64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    AttnArgs f = a;
    f.dq_fallback = 1;
    if (a.k_rows)
      hipLaunchKernelGGL((k_bwd_dq_bf16<MODE, D, BS, true>), dim3((unsigned)(a.BH * a.nq)), dim3(BS / 32 * 64), 0, s, f);
    else
      hipLaunchKernelGGL((k_bwd_dq_bf16<MODE, D, BS, false>), dim3((unsigned)(a.BH * a.nq)), dim3(BS / 32 * 64), 0, s, f);
    return hipGetLastError();
  }
  return hipSuccess;
}

#define SCFA_DISPATCH_B(FN, a, mode, s)                                                     \
  do {                                                                                      \
    const int key = (mode) * 4 + ((a).d == 128 ? 2 : 0) + ((a).block == 128 ? 1 : 0);       \
    switch (key) {                                                                          \
      case 0: return FN<kDense, 64, 64>(a, part, s);                                            \
      case 1: return FN<kDense, 64, 128>(a, part, s);                                             \
      case 2: return FN<kDense, 128, 64>(a, part, s);                                             \
      case 3: return FN<kDense, 128, 128>(a, part, s);                                            \
      case 4: return FN<kQK, 64, 64>(a, part, s);                                                 \
      case 5: return FN<kQK, 64, 128>(a, part, s);                                                \
      case 6: return FN<kQK, 128, 64>(a, part, s);                                                \
      case 7: return FN<kQK, 128, 128>(a, part, s);                                               \
      case 8: return FN<kHash, 64, 64>(a, part, s);                                               \
      case 9: return FN<kHash, 64, 128>(a, part, s);                                              \
      case 10: return FN<kHash, 128, 64>(a, part, s);                                             \
      case 11: return FN<kHash, 128, 128>(a, part, s);                                            \
      default: return hipErrorInvalidValue;                                                 \
    }                                                                                       \
  } while (0)

hipError_t launch_attn_bwd_bf16(const AttnArgs &a, int mode, int part, hipStream_t s) {
  if (a.BH == 0) return hipSuccess;
  SCFA_DISPATCH_B(run_bwd_bf16, a, mode, s);
}

hipError_t launch_attn_bwd_f32(const AttnArgs &a, int mode, int part, hipStream_t s) {
  if (a.BH == 0) return hipSuccess;
  SCFA_DISPATCH_B(run_bwd_f32, a, mode, s);
}

hipError_t launch_attn_bwd_ds_bf16(const AttnArgs &a, int mode, int part, hipStream_t s) {
  if (a.BH == 0) return hipSuccess;
  const int key = (mode == kHash ? 4 : 0) + (a.d == 128 ? 2 : 0) + (a.block == 128 ? 1 : 0);
  if (mode == kDense) return hipErrorInvalidValue;  // no lists, no slots
  switch (key) {
    case 0: return run_bwd_ds_bf16<kQK, 64, 64>(a, part, s);
    case 1: return run_bwd_ds_bf16<kQK, 64, 128>(a, part, s);
    case 2: return run_bwd_ds_bf16<kQK, 128, 64>(a, part, s);
    case 3: return run_bwd_ds_bf16<kQK, 128, 128>(a, part, s);
    case 4: return run_bwd_ds_bf16<kHash, 64, 64>(a, part, s);
    case 5: return run_bwd_ds_bf16<kHash, 64, 128>(a, part, s);
    case 6: return run_bwd_ds_bf16<kHash, 128, 64>(a, part, s);
    case 7: return run_bwd_ds_bf16<kHash, 128, 128>(a, part, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_bwd_prep(const AttnArgs &a, hipStream_t s) {
  const long long lanes = 2ll * a.BH * a.Tq;
  if (lanes == 0) return hipSuccess;
  const dim3 grid((unsigned)((lanes + 255) / 256));
  if (a.d == 64) hipLaunchKernelGGL(k_bwd_prep<64>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_bwd_prep<128>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace scfa
