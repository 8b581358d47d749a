// Host-side interface between the C ABI (api.cpp) and the kernel translation
// units.  Every launcher enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace scfa {

// Attention modes: dense causal (positions 0..T-1), QK-sparse, Hash-sparse.
enum Mode { kDense = 0, kQK = 1, kHash = 2 };

struct AttnArgs {
  // inputs [BH, T, d]
  const void *q, *k, *v;
  const void *o, *dout;  // backward only
  const float *lse;      // backward only [BH, Tq]
  // outputs
  void *out_o;
  float *out_lse;
  void *dq, *dk, *dv;
  float *delta;  // backward scratch [BH, Tq]: rowsum(dO * O)
  // positions / buckets [BH, T] (idx NULL => dense causal)
  const int32_t *q_idx, *k_idx, *q_hash, *k_hash;
  // optional row indirection [BH, T]: row i of Q (dO) is row q_rows[i] of q (dout), row j of K, V is
  // row k_rows[j] of k, v (NULL = identity); outputs stay indexed by i and j
  const int32_t *q_rows, *k_rows;
  // Rows per head of the caller's tensors: q and dout hold Tqs rows per head, k and v Tks (with row
  // indirection these may differ from the view's Tq, Tk, e.g. full-length tensors read at the kept
  // positions); the q-side outputs (o, lse, dq, and the backward's o / lse inputs) hold Tqo rows per
  // head and the k-side ones (dk, dv) Tko: Tqs / Tks with orig_rows, else Tq / Tk.
  int Tqs, Tks, Tqo, Tko;
  // live-tile lists (NULL in dense mode)
  const int32_t *row_cnt, *row_list;  // [BH, nq], [BH, nq, nk]
  const int32_t *col_cnt, *col_list;  // [BH, nk], [BH, nk, nq]
  int BH, Tq, Tk, nq, nk, d, block;
  float scale;
  int no_prune, force_mask;
  // Stored dS (bf16 tiles [block keys][block queries], one per live tile, in the
  // slots of the tile-slot numbering): the dK/dV kernel writes key block c's
  // tiles to slots col_base[c] + t, the dQ kernel reads the tiles named by
  // row_slot.  ds_tiles is the buffer's capacity; when the total tile count
  // col_base[BH*nk] exceeds it, nothing is stored and the recomputing dQ kernel
  // (dq_fallback) runs instead of the stored-dS one.
  void *ds;
  const int32_t *row_slot, *col_base;
  long long ds_tiles;
  int dq_fallback;
  // With row indirection: outputs (O, lse, dQ, dK, dV) and the backward's o / lse
  // inputs are indexed by the caller's rows (q_rows[i], k_rows[j]) instead of the
  // view's rows i, j; delta stays indexed by the view.
  int orig_rows;
  // Packed ragged heads: head bh's query rows are q_off[bh] .. q_off[bh+1]-1 of
  // the packed tensors (k_off for keys), at most Tq (Tk) of them; NULL = every
  // head has Tq (Tk) rows at bh*Tq.  delta_half is the offset of delta's second
  // half (lse * log2 e): BH*Tq, or the packed query row count.
  const int32_t *q_off, *k_off;
  long long delta_half;
  long long q_total, k_total;  // packed rows of the ragged-head tensors (bounds for the offsets)
};

// Packed ragged heads: rebase every per-head pointer of head bh so that the
// kernels' usual addressing (row bh*Tq + i) lands on packed row q_off[bh] + i,
// and set Tq, Tk (and the caller row counts) to this head's lengths (clamped into [0, max]).  esize is the
// element size of the [rows, d] tensors.  Returns whether the head is ragged.
__device__ __forceinline__ bool varlen_head(AttnArgs &a, int bh, int esize) {
  if (a.q_off == nullptr) return false;
  // first row clamped into [0, total], length into [0, min(max, total - first)]: malformed offsets
  // give wrong results, but every access stays inside the packed tensors
  const long long q0 = min(max((long long)a.q_off[bh], 0ll), a.q_total);
  const long long k0 = min(max((long long)a.k_off[bh], 0ll), a.k_total);
  const int Tq = (int)min(max((long long)a.q_off[bh + 1] - q0, 0ll), min((long long)a.Tq, a.q_total - q0));
  const int Tk = (int)min(max((long long)a.k_off[bh + 1] - k0, 0ll), min((long long)a.Tk, a.k_total - k0));
  const long long sq = q0 - (long long)bh * Tq, sk = k0 - (long long)bh * Tk;  // row shifts
  const long long bq = sq * a.d * esize, bk = sk * a.d * esize;                   // byte shifts of [rows, d]
  auto mv = [](const void *p, long long bytes) { return p ? static_cast<const char *>(p) + bytes : nullptr; };
  auto mvw = [](void *p, long long bytes) { return p ? static_cast<char *>(p) + bytes : nullptr; };
  a.q = mv(a.q, bq);
  a.o = mv(a.o, bq);
  a.dout = mv(a.dout, bq);
  a.out_o = mvw(a.out_o, bq);
  a.dq = mvw(a.dq, bq);
  a.k = mv(a.k, bk);
  a.v = mv(a.v, bk);
  a.dk = mvw(a.dk, bk);
  a.dv = mvw(a.dv, bk);
  if (a.lse) a.lse += sq;
  if (a.out_lse) a.out_lse += sq;
  if (a.delta) a.delta += sq;
  if (a.q_idx) a.q_idx += sq;
  if (a.q_hash) a.q_hash += sq;
  if (a.q_rows) a.q_rows += sq;
  if (a.k_idx) a.k_idx += sk;
  if (a.k_hash) a.k_hash += sk;
  if (a.k_rows) a.k_rows += sk;
  a.Tq = a.Tqs = a.Tqo = Tq;  // ragged heads have no row indirection: every tensor is in view order
  a.Tk = a.Tks = a.Tko = Tk;
  return true;
}

// Caller row of view query row i (view key row j): through the permutation when
// outputs go to the caller's rows, clamped into the head.
__device__ __forceinline__ int out_row_q(const AttnArgs &a, size_t bh, int i) {
  return a.orig_rows ? min(max(a.q_rows[bh * a.Tq + i], 0), a.Tqs - 1) : i;
}
__device__ __forceinline__ int out_row_k(const AttnArgs &a, size_t bh, int j) {
  return a.orig_rows ? min(max(a.k_rows[bh * a.Tk + j], 0), a.Tks - 1) : j;
}

// Row gather / scatter: [BH, Ts, row] <-> [BH, Td, row], rows of ppr 16-byte
// pieces, index [BH, Td] (gather) or [BH, Ts] (scatter).
struct RowArgs {
  const void *src;
  const int32_t *index;
  void *dst;
  int BH, Ts, Td, ppr;
};

// Bucket segments of a block (exact tile test): one int4 record (bucket, min
// position, max position, 0) per distinct bucket among the block's real rows,
// in ascending bucket order, `block` record slots per block; the number of
// records is in the block's count entry.
struct MetaArgs {
  const int32_t *q_idx, *k_idx, *q_hash, *k_hash;
  const int32_t *q_off, *k_off;  // packed ragged heads (NULL = fixed Tq, Tk per head), as in AttnArgs
  long long q_total, k_total;    // their packed row counts
  int32_t *q_stats, *k_stats;  // [BH, nq, 4], [BH, nk, 4]
  int32_t *q_segs, *k_segs;    // [BH, nq, block, 4], [BH, nk, block, 4]; NULL = range rule only
  int32_t *q_nseg, *k_nseg;    // [BH, nq], [BH, nk] record counts (with the segments)
  int32_t *row_cnt, *row_list, *col_cnt, *col_list;
  int BH, Tq, Tk, nq, nk, block;
};

// Workspace slices are 256-byte aligned.
constexpr size_t kWsAlign = 256;
inline size_t ws_round(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Workspace bytes of the exact tile test's segments (records and counts).
inline size_t meta_seg_bytes(size_t BH, size_t nq, size_t nk, int block) {
  return ws_round(BH * nq * block * 16) + ws_round(BH * nk * block * 16) + ws_round(BH * nq * 4) +
         ws_round(BH * nk * 4);
}

struct LshArgs {
  const void *x;
  // Row indirection (nullable): token t of sequence bh is row x_rows[bh*T + t] (clamped into
  // [0, Tx)) of x, which has Tx rows per head; NULL = row t, Tx = T.
  const int32_t *x_rows;
  int Tx;
  const int32_t *idx;  // nullable
  const float *R;      // [H, d, nb/2]
  int nb, B, H, T, d, dtype;
  int idx_ascending;
  int32_t *hash_sorted, *idx_sorted, *perm;
  void *x_sorted;
  const void *companion;
  void *companion_sorted;
  // workspace pieces
  int32_t *hash;            // [BH, T]
  int32_t *hist;            // [BH, nbins, nchunks]
  int32_t *tmp_idx[2];      // [BH, T] ping-pong (radix passes over idx)
  int32_t *tmp_src[2];
  double *R64;              // [H, lsh_r64_cols(nb) / lsh_col_group(nb), d, lsh_col_group(nb)] float64 R (float32 inputs)
  // matrix-core projection (bf16 inputs)
  void *Rf;                 // [H, lsh_col_tiles(nb), 3, d/16, 64] uint4: R split into three bf16 terms
  float *colnorm;           // [H, nb/2] upper bounds of the column 2-norms of R
  int32_t *fb_count;        // tokens whose bucket the matrix-core pass could not certify
  int32_t *fb_list;         // [BH * T] their indices (b*H + h) * T + t
  int32_t *scan_tmp;        // [2, BH, nbins] row totals and digit offsets of the two-level scan
};

hipError_t launch_block_meta(const MetaArgs &a, bool with_cols, hipStream_t s);
// col_base [BH*nk + 1] (exclusive scan of the column counts, total last) and
// row_slot [BH, nq, nk] (slot of each row-list entry's tile).
hipError_t launch_tile_slots(const int32_t *row_cnt, const int32_t *row_list, const int32_t *col_cnt,
                             const int32_t *col_list, int BH, int nq, int nk, int32_t *col_base, int32_t *row_slot,
                             hipStream_t s);

// Sets the calling thread's scfa_last_error() message and returns `code`.
int report_error(int code, const char *msg);

hipError_t launch_gather_rows(const RowArgs &r, hipStream_t s);
hipError_t launch_scatter_rows(const RowArgs &r, bool zero_fill, hipStream_t s);
// dst[bh, index[bh, i]] = 0 for i < Ts (src unused)
hipError_t launch_zero_rows(const RowArgs &r, hipStream_t s);
hipError_t launch_attn_fwd_bf16(const AttnArgs &a, int mode, hipStream_t s);
hipError_t launch_attn_fwd_f32(const AttnArgs &a, int mode, hipStream_t s);
// part: bit 0 = dQ (+ D = rowsum(dO * O)), bit 1 = dK/dV (reads D).
hipError_t launch_attn_bwd_bf16(const AttnArgs &a, int mode, int part, hipStream_t s);
hipError_t launch_attn_bwd_f32(const AttnArgs &a, int mode, int part, hipStream_t s);
// Backward preprocess: delta[0] = rowsum(dO * O), delta[1] = lse * log2 e (bf16).
hipError_t launch_attn_bwd_prep(const AttnArgs &a, hipStream_t s);
// Stored-dS backward (bf16, pruned modes): part 2 = dK/dV writing dS tiles,
// part 1 = dQ from the dS tiles (+ the guarded recomputing fallback).
hipError_t launch_attn_bwd_ds_bf16(const AttnArgs &a, int mode, int part, hipStream_t s);

hipError_t launch_lsh_bucket_sort(const LshArgs &a, hipStream_t s);

// Sizes shared by the API's workspace carving and the sort launcher.
constexpr int kSortChunk = 256;  // tokens per counting-sort work group (one per thread)
inline int sort_bins(int nb, bool idx_passes) { return idx_passes ? (nb > 256 ? nb : 256) : nb; }
inline int sort_chunks(int T) { return (T + kSortChunk - 1) / kSortChunk; }
// LSH projection: columns per register group, and the float64 copy of R's
// row length (nb/2 padded with zeros to a whole number of groups).
inline int lsh_col_group(int nb) { return nb / 2 <= 8 ? 8 : nb / 2 <= 16 ? 16 : 32; }
inline int lsh_r64_cols(int nb) {
  const int g = lsh_col_group(nb);
  return (nb / 2 + g - 1) / g * g;
}
// Matrix-core projection: 32-column tiles of R and the bytes of its bf16 split.
inline int lsh_col_tiles(int nb) { return (nb / 2 + 31) / 32; }
inline size_t lsh_frag_bytes(int H, int d, int nb) { return (size_t)H * lsh_col_tiles(nb) * 3 * (d / 16) * 64 * 16; }

}  // namespace scfa
