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
// block of BS rows); wave w owns queries 32w..32w+31.  Each live key block is
// streamed through LDS in 64-key chunks: K row-major, V transposed.  The
// kernel computes S^T = K Q^T so that every lane owns ONE query column: the
// row max and row sum of the online softmax are in-lane except for a single
// exchange with lane l^32, the O^T accumulator rescale is in-lane, and the
// S^T registers feed the O^T += V^T P^T product directly as B operands.
//
// fp32 kernel: one thread per query, plain fp32 FMAs over 32-key LDS chunks.
#include "scfa_device.hpp"
#include "scfa_internal.hpp"

namespace scfa {

// Live list of a query block: returns the count; entry t is read by tile_at.
struct RowList {
  int n;
  const int32_t *list;
};

template <int MODE, int BS>
__device__ __forceinline__ RowList row_list(const AttnArgs &a, int bh, int qb) {
  RowList r;
  r.list = nullptr;
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

// Key block of entry t and whether the whole tile is admissible (mask-free).
template <int MODE, int BS>
__device__ __forceinline__ void tile_at(const AttnArgs &a, const RowList &rl, int t, int qb, int &kb, bool &free) {
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

template <int MODE, int D, int BS>
__global__ __launch_bounds__(BS / 32 * 64) void k_fwd_bf16(AttnArgs a) {
  constexpr int NW = BS / 32;
  constexpr int NT = NW * 64;
  constexpr int NCH = BS / kChunk;
  __shared__ __attribute__((aligned(16))) uint16_t sK[kChunk * (D + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * kTPad];
  __shared__ __attribute__((aligned(16))) int sKidx[kChunk];
  __shared__ __attribute__((aligned(16))) int sKhash[kChunk];

  const int bh = blockIdx.x / a.nq;
  const int qb = blockIdx.x % a.nq;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int qrow = qb * BS + 32 * w + col;
  const bool qvalid = qrow < a.Tq;
  const uint16_t *Q = static_cast<const uint16_t *>(a.q) + (size_t)bh * a.Tq * D;
  const uint16_t *K = static_cast<const uint16_t *>(a.k) + (size_t)bh * a.Tk * D;
  const uint16_t *V = static_cast<const uint16_t *>(a.v) + (size_t)bh * a.Tk * D;

  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    qf[kk] = as_bf16x8(qvalid ? ld16(Q + (size_t)qrow * D + 16 * kk + 8 * half) : make_uint4(0, 0, 0, 0));
  int my_idx = kIdxTailQ, my_hash = 0;
  if (qvalid) {
    my_idx = MODE == kDense ? qrow : a.q_idx[(size_t)bh * a.Tq + qrow];
    if (MODE == kHash) my_hash = a.q_hash[(size_t)bh * a.Tq + qrow];
  }

  const RowList rl = row_list<MODE, BS>(a, bh, qb);
  const float c = a.scale * kLog2e;
  float m = -INFINITY, l = 0.f;
  f32x16 acc[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;

  for (int t = 0; t < rl.n; ++t) {
    int kb;
    bool free;
    tile_at<MODE, BS>(a, rl, t, qb, kb, free);
    if (kb >= a.nk) continue;  // entries outside the sequence are skipped
#pragma unroll 1
    for (int ch = 0; ch < NCH; ++ch) {
      const int k0 = kb * BS + ch * kChunk;
      const int kvalid = min(kChunk, a.Tk - k0);
      if (kvalid <= 0) break;
      const bool nomask = free && kvalid == kChunk;
      __syncthreads();
      stage_rows<D, NT>(sK, K, k0, kvalid);
      stage_transposed<D, NT>(sVt, V, k0, kvalid);
      if (MODE != kDense && !nomask) {
        for (int r = threadIdx.x; r < kChunk; r += NT) {
          sKidx[r] = r < kvalid ? a.k_idx[(size_t)bh * a.Tk + k0 + r] : kIdxTailK;
          if (MODE == kHash) sKhash[r] = r < kvalid ? a.k_hash[(size_t)bh * a.Tk + k0 + r] : 0;
        }
      }
      __syncthreads();

      f32x16 s[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[sub][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) s[sub] = mfma32(lds_a_rows<D>(sK, 32 * sub + col, kk, half), qf[kk], s[sub]);
      }
      if (!nomask) {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int kr = 32 * sub + 8 * g + 4 * half;
            int4 ki, kh = make_int4(0, 0, 0, 0);
            if (MODE == kDense) {
              ki.x = kr + 0 < kvalid ? k0 + kr + 0 : kIdxTailK;
              ki.y = kr + 1 < kvalid ? k0 + kr + 1 : kIdxTailK;
              ki.z = kr + 2 < kvalid ? k0 + kr + 2 : kIdxTailK;
              ki.w = kr + 3 < kvalid ? k0 + kr + 3 : kIdxTailK;
            } else {
              ki = *reinterpret_cast<const int4 *>(sKidx + kr);
              if (MODE == kHash) kh = *reinterpret_cast<const int4 *>(sKhash + kr);
            }
            const int kiv[4] = {ki.x, ki.y, ki.z, ki.w};
            const int khv[4] = {kh.x, kh.y, kh.z, kh.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool ok = kiv[e] <= my_idx && (MODE != kHash || khv[e] == my_hash);
              if (!ok) s[sub][4 * g + e] = -INFINITY;
            }
          }
      }

      float mx = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sub][r]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f((m - m_use) * c);
      const float mc = m_use * c;
      float rs = 0.f;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[sub][r], c, -mc));
          s[sub][r] = p;
          rs += p;
        }
      l = l * alpha + rs;
      m = m_new;
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mt][r] *= alpha;

#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const bf16x8 pb = c_regs_to_bf16x8(s[sub], t2);
#pragma unroll
          for (int mt = 0; mt < D / 32; ++mt)
            acc[mt] = mfma32(lds_a_trans(sVt, 32 * mt + col, 32 * sub + 16 * t2, half), pb, acc[mt]);
        }
    }
  }

  const float lt = pair_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qvalid) {
    uint16_t *O = static_cast<uint16_t *>(a.out_o) + ((size_t)bh * a.Tq + qrow) * D;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mt + 8 * g + 4 * half;
        const uint2 val = make_uint2(pack_bf16x2(acc[mt][4 * g] * inv, acc[mt][4 * g + 1] * inv),
                                     pack_bf16x2(acc[mt][4 * g + 2] * inv, acc[mt][4 * g + 3] * inv));
        *reinterpret_cast<uint2 *>(O + d0) = val;
      }
    if (half == 0) a.out_lse[(size_t)bh * a.Tq + qrow] = lt > 0.f ? m * a.scale + logf(lt) : -INFINITY;
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
  const RowList rl = row_list<MODE, BS>(a, bh, qb);
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
  hipLaunchKernelGGL((k_fwd_bf16<MODE, D, BS>), dim3((unsigned)(a.BH * a.nq)), dim3(BS / 32 * 64), 0, s, a);
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
