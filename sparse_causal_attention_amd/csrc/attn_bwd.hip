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
#include "scfa_device.hpp"
#include "scfa_internal.hpp"

namespace scfa {

struct List {
  int n;
  int first;
  const int32_t *list;
};

template <int MODE, int BS>
__device__ __forceinline__ List row_list_b(const AttnArgs &a, int bh, int qb) {
  List r{0, 0, nullptr};
  if (a.no_prune) {
    r.n = a.nk;
  } else if (MODE == kDense) {
    const int qmax = min((qb + 1) * BS, a.Tq) - 1;
    r.n = min(a.nk, qmax / BS + 1);
  } else {
    r.n = min(a.row_cnt[(size_t)bh * a.nq + qb], a.nk);  // malformed counts never overrun the row
    r.list = a.row_list + ((size_t)bh * a.nq + qb) * a.nk;
  }
  return r;
}

template <int MODE, int BS>
__device__ __forceinline__ void row_tile(const AttnArgs &a, const List &rl, int t, int qb, int &kb, bool &free) {
  if (a.no_prune) {
    kb = t;
    free = false;
  } else if (MODE == kDense) {
    kb = t;
    free = min((kb + 1) * BS, a.Tk) - 1 <= qb * BS;
  } else {
    const int e = rl.list[t];
    kb = e & 0x7fffffff;
    free = e < 0;
  }
  if (a.force_mask) free = false;
}

template <int MODE, int BS>
__device__ __forceinline__ List col_list_b(const AttnArgs &a, int bh, int kb) {
  List r{0, 0, nullptr};
  if (a.no_prune) {
    r.n = a.nq;
  } else if (MODE == kDense) {
    // live(i, kb) iff min((i+1)*BS, Tq) - 1 >= kb*BS, i.e. i >= kb when kb*BS < Tq
    r.first = kb;
    r.n = kb * BS < a.Tq ? a.nq - kb : 0;
  } else {
    r.n = min(a.col_cnt[(size_t)bh * a.nk + kb], a.nq);
    r.list = a.col_list + ((size_t)bh * a.nk + kb) * a.nq;
  }
  return r;
}

template <int MODE, int BS>
__device__ __forceinline__ void col_tile(const AttnArgs &a, const List &cl, int t, int kb, int &qb, bool &free) {
  if (a.no_prune) {
    qb = t;
    free = false;
  } else if (MODE == kDense) {
    qb = cl.first + t;
    free = min((kb + 1) * BS, a.Tk) - 1 <= qb * BS;
  } else {
    const int e = cl.list[t];
    qb = e & 0x7fffffff;
    free = e < 0;
  }
  if (a.force_mask) free = false;
}

// ---------------------------------------------------------------------------
// bf16 dQ (+ D) kernel
// ---------------------------------------------------------------------------
template <int MODE, int D, int BS>
__global__ __launch_bounds__(BS / 32 * 64) void k_bwd_dq_bf16(AttnArgs a) {
  constexpr int NT = BS / 32 * 64;
  constexpr int NCH = BS / kChunk;
  __shared__ __attribute__((aligned(16))) uint16_t sK[kChunk * (D + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t sKt[D * kTPad];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kChunk * (D + 8)];
  __shared__ __attribute__((aligned(16))) int sKidx[kChunk];
  __shared__ __attribute__((aligned(16))) int sKhash[kChunk];

  const int bh = blockIdx.x / a.nq;
  const int qb = blockIdx.x % a.nq;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int qrow = qb * BS + 32 * w + col;
  const bool qvalid = qrow < a.Tq;
  const size_t qoff = (size_t)bh * a.Tq;
  const uint16_t *Q = static_cast<const uint16_t *>(a.q) + qoff * D;
  const uint16_t *dO = static_cast<const uint16_t *>(a.dout) + qoff * D;
  const uint16_t *O = static_cast<const uint16_t *>(a.o) + qoff * D;
  const uint16_t *K = static_cast<const uint16_t *>(a.k) + (size_t)bh * a.Tk * D;
  const uint16_t *V = static_cast<const uint16_t *>(a.v) + (size_t)bh * a.Tk * D;

  bf16x8 qf[D / 16], dof[D / 16];
  float dsum = 0.f;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const size_t off = (size_t)qrow * D + 16 * kk + 8 * half;
    const uint4 zq = make_uint4(0, 0, 0, 0);
    const uint4 uq = qvalid ? ld16(Q + off) : zq;
    const uint4 ud = qvalid ? ld16(dO + off) : zq;
    const uint4 uo = qvalid ? ld16(O + off) : zq;
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
  if (qvalid && half == 0) a.delta[qoff + qrow] = dsum;
  const float lse2 = qvalid ? a.lse[qoff + qrow] * kLog2e : INFINITY;
  int my_idx = kIdxTailQ, my_hash = 0;
  if (qvalid) {
    my_idx = MODE == kDense ? qrow : a.q_idx[qoff + qrow];
    if (MODE == kHash) my_hash = a.q_hash[qoff + qrow];
  }
  const float c = a.scale * kLog2e;
  f32x16 dqa[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[mt][r] = 0.f;

  const List rl = row_list_b<MODE, BS>(a, bh, qb);
  for (int t = 0; t < rl.n; ++t) {
    int kb;
    bool free;
    row_tile<MODE, BS>(a, rl, t, qb, kb, free);
    if (kb >= a.nk) continue;  // entries outside the sequence are skipped
#pragma unroll 1
    for (int ch = 0; ch < NCH; ++ch) {
      const int k0 = kb * BS + ch * kChunk;
      const int kvalid = min(kChunk, a.Tk - k0);
      if (kvalid <= 0) break;
      const bool nomask = free && kvalid == kChunk;
      __syncthreads();
      stage_rows<D, NT>(sK, K, k0, kvalid);
      stage_transposed<D, NT>(sKt, K, k0, kvalid);
      stage_rows<D, NT>(sV, V, k0, kvalid);
      if (MODE != kDense && !nomask) {
        for (int r = threadIdx.x; r < kChunk; r += NT) {
          sKidx[r] = r < kvalid ? a.k_idx[(size_t)bh * a.Tk + k0 + r] : kIdxTailK;
          if (MODE == kHash) sKhash[r] = r < kvalid ? a.k_hash[(size_t)bh * a.Tk + k0 + r] : 0;
        }
      }
      __syncthreads();

      f32x16 s[2], dp[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[sub][r] = 0.f;
          dp[sub][r] = 0.f;
        }
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          s[sub] = mfma32(lds_a_rows<D>(sK, 32 * sub + col, kk, half), qf[kk], s[sub]);
          dp[sub] = mfma32(lds_a_rows<D>(sV, 32 * sub + col, kk, half), dof[kk], dp[sub]);
        }
      }
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int kr = 32 * sub + 8 * g + 4 * half;
          int kiv[4] = {0, 0, 0, 0}, khv[4] = {0, 0, 0, 0};
          if (!nomask) {
            if (MODE == kDense) {
#pragma unroll
              for (int e = 0; e < 4; ++e) kiv[e] = kr + e < kvalid ? k0 + kr + e : kIdxTailK;
            } else {
              const int4 ki = *reinterpret_cast<const int4 *>(sKidx + kr);
              kiv[0] = ki.x; kiv[1] = ki.y; kiv[2] = ki.z; kiv[3] = ki.w;
              if (MODE == kHash) {
                const int4 kh = *reinterpret_cast<const int4 *>(sKhash + kr);
                khv[0] = kh.x; khv[1] = kh.y; khv[2] = kh.z; khv[3] = kh.w;
              }
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            const bool ok = nomask || (kiv[e] <= my_idx && (MODE != kHash || khv[e] == my_hash));
            const float p = ok ? __builtin_amdgcn_exp2f(fmaf(s[sub][r], c, -lse2)) : 0.f;
            s[sub][r] = p * (dp[sub][r] - dsum);
          }
        }
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const bf16x8 db = c_regs_to_bf16x8(s[sub], t2);
#pragma unroll
          for (int mt = 0; mt < D / 32; ++mt)
            dqa[mt] = mfma32(lds_a_trans(sKt, 32 * mt + col, 32 * sub + 16 * t2, half), db, dqa[mt]);
        }
    }
  }

  if (qvalid) {
    uint16_t *dQ = static_cast<uint16_t *>(a.dq) + (qoff + qrow) * D;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mt + 8 * g + 4 * half;
        *reinterpret_cast<uint2 *>(dQ + d0) =
            make_uint2(pack_bf16x2(dqa[mt][4 * g] * a.scale, dqa[mt][4 * g + 1] * a.scale),
                       pack_bf16x2(dqa[mt][4 * g + 2] * a.scale, dqa[mt][4 * g + 3] * a.scale));
      }
  }
}

// ---------------------------------------------------------------------------
// bf16 dK / dV kernel
// ---------------------------------------------------------------------------
template <int MODE, int D, int BS>
__global__ __launch_bounds__(BS / 32 * 64) void k_bwd_dkdv_bf16(AttnArgs a) {
  constexpr int NT = BS / 32 * 64;
  constexpr int NCH = BS / kChunk;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[kChunk * (D + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t sQt[D * kTPad];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[kChunk * (D + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t sdOt[D * kTPad];
  __shared__ __attribute__((aligned(16))) float sLse[kChunk];
  __shared__ __attribute__((aligned(16))) float sDel[kChunk];
  __shared__ __attribute__((aligned(16))) int sQidx[kChunk];
  __shared__ __attribute__((aligned(16))) int sQhash[kChunk];

  const int bh = blockIdx.x / a.nk;
  const int kb = blockIdx.x % a.nk;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int krow = kb * BS + 32 * w + col;
  const bool kvalid_row = krow < a.Tk;
  const size_t koff = (size_t)bh * a.Tk;
  const size_t qoff = (size_t)bh * a.Tq;
  const uint16_t *Q = static_cast<const uint16_t *>(a.q) + qoff * D;
  const uint16_t *dO = static_cast<const uint16_t *>(a.dout) + qoff * D;
  const uint16_t *K = static_cast<const uint16_t *>(a.k) + koff * D;
  const uint16_t *V = static_cast<const uint16_t *>(a.v) + koff * D;

  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const size_t off = (size_t)krow * D + 16 * kk + 8 * half;
    kf[kk] = as_bf16x8(kvalid_row ? ld16(K + off) : make_uint4(0, 0, 0, 0));
    vf[kk] = as_bf16x8(kvalid_row ? ld16(V + off) : make_uint4(0, 0, 0, 0));
  }
  int my_idx = kIdxTailK, my_hash = 0;
  if (kvalid_row) {
    my_idx = MODE == kDense ? krow : a.k_idx[koff + krow];
    if (MODE == kHash) my_hash = a.k_hash[koff + krow];
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

  const List cl = col_list_b<MODE, BS>(a, bh, kb);
  for (int t = 0; t < cl.n; ++t) {
    int qb;
    bool free;
    col_tile<MODE, BS>(a, cl, t, kb, qb, free);
    if (qb >= a.nq) continue;
#pragma unroll 1
    for (int ch = 0; ch < NCH; ++ch) {
      const int q0 = qb * BS + ch * kChunk;
      const int qv = min(kChunk, a.Tq - q0);
      if (qv <= 0) break;
      // Query rows past Tq carry lse = +inf (P = 0); key rows past Tk only
      // pollute their own, never stored, columns.  So a mask-free tile needs
      // no mask even when either block is partial.
      const bool nomask = free;
      __syncthreads();
      stage_rows<D, NT>(sQ, Q, q0, qv);
      stage_transposed<D, NT>(sQt, Q, q0, qv);
      stage_rows<D, NT>(sdO, dO, q0, qv);
      stage_transposed<D, NT>(sdOt, dO, q0, qv);
      for (int r = threadIdx.x; r < kChunk; r += NT) {
        const bool ok = r < qv;
        sLse[r] = ok ? a.lse[qoff + q0 + r] * kLog2e : INFINITY;
        sDel[r] = ok ? a.delta[qoff + q0 + r] : 0.f;
        if (MODE != kDense) sQidx[r] = ok ? a.q_idx[qoff + q0 + r] : kIdxTailQ;
        else sQidx[r] = ok ? q0 + r : kIdxTailQ;
        if (MODE == kHash) sQhash[r] = ok ? a.q_hash[qoff + q0 + r] : 0;
      }
      __syncthreads();

      f32x16 s[2], dp[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[sub][r] = 0.f;
          dp[sub][r] = 0.f;
        }
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          s[sub] = mfma32(lds_a_rows<D>(sQ, 32 * sub + col, kk, half), kf[kk], s[sub]);
          dp[sub] = mfma32(lds_a_rows<D>(sdO, 32 * sub + col, kk, half), vf[kk], dp[sub]);
        }
      }
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qr = 32 * sub + 8 * g + 4 * half;
          const float4 l4 = *reinterpret_cast<const float4 *>(sLse + qr);
          const float4 d4 = *reinterpret_cast<const float4 *>(sDel + qr);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
          int qiv[4] = {0, 0, 0, 0}, qhv[4] = {0, 0, 0, 0};
          if (!nomask) {
            const int4 qi = *reinterpret_cast<const int4 *>(sQidx + qr);
            qiv[0] = qi.x; qiv[1] = qi.y; qiv[2] = qi.z; qiv[3] = qi.w;
            if (MODE == kHash) {
              const int4 qh = *reinterpret_cast<const int4 *>(sQhash + qr);
              qhv[0] = qh.x; qhv[1] = qh.y; qhv[2] = qh.z; qhv[3] = qh.w;
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            const bool ok = nomask || (my_idx <= qiv[e] && (MODE != kHash || qhv[e] == my_hash));
            const float p = ok ? __builtin_amdgcn_exp2f(fmaf(s[sub][r], c, -lv[e])) : 0.f;
            s[sub][r] = p;
            dp[sub][r] = p * (dp[sub][r] - dv4[e]);
          }
        }
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const bf16x8 pb = c_regs_to_bf16x8(s[sub], t2);
          const bf16x8 db = c_regs_to_bf16x8(dp[sub], t2);
#pragma unroll
          for (int mt = 0; mt < D / 32; ++mt) {
            dva[mt] = mfma32(lds_a_trans(sdOt, 32 * mt + col, 32 * sub + 16 * t2, half), pb, dva[mt]);
            dka[mt] = mfma32(lds_a_trans(sQt, 32 * mt + col, 32 * sub + 16 * t2, half), db, dka[mt]);
          }
        }
    }
  }

  if (kvalid_row) {
    uint16_t *dK = static_cast<uint16_t *>(a.dk) + (koff + krow) * D;
    uint16_t *dV = static_cast<uint16_t *>(a.dv) + (koff + krow) * D;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mt + 8 * g + 4 * half;
        *reinterpret_cast<uint2 *>(dK + d0) =
            make_uint2(pack_bf16x2(dka[mt][4 * g] * a.scale, dka[mt][4 * g + 1] * a.scale),
                       pack_bf16x2(dka[mt][4 * g + 2] * a.scale, dka[mt][4 * g + 3] * a.scale));
        *reinterpret_cast<uint2 *>(dV + d0) = make_uint2(pack_bf16x2(dva[mt][4 * g], dva[mt][4 * g + 1]),
                                                         pack_bf16x2(dva[mt][4 * g + 2], dva[mt][4 * g + 3]));
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
  const List rl = row_list_b<MODE, BS>(a, bh, qb);
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
  const List cl = col_list_b<MODE, BS>(a, bh, kb);
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
    hipLaunchKernelGGL((k_bwd_dq_bf16<MODE, D, BS>), dim3((unsigned)(a.BH * a.nq)), dim3(BS / 32 * 64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((part & 2) && a.nk > 0) {
    hipLaunchKernelGGL((k_bwd_dkdv_bf16<MODE, D, BS>), dim3((unsigned)(a.BH * a.nk)), dim3(BS / 32 * 64), 0, s, a);
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

}  // namespace scfa
