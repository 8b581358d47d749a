/*
 * scfa.h - C ABI of the MI355X (gfx950) sparse causal flash attention library.
 *
 * Sparse Causal Flash Attention (SCFA) is tiled, online-softmax causal
 * attention over COMPACTED tensors: rows of Q, K and V may have been dropped
 * or reordered, and every row carries its ORIGINAL position (q_idx, k_idx) and,
 * in Hash-sparse mode, an LSH bucket id (q_hash, k_hash).  Source: the
 * deep-paper.org summary of arXiv 2306.01160, "Faster Causal Attention Over
 * Large Sequences Through Sparse Flash Attention" (page title
 * "超越 FlashAttention：利用动态稀疏性让 Transformer 再提速"), sections
 * "SCFA solution > 1. QK-Sparse" and "2. Hash-Sparse".
 *
 * What every attention entry point computes, per (batch b, head h):
 *   valid(i, j) = k_idx[j] <= q_idx[i]                 (causality on original
 *                                                       positions, "1. QK-Sparse"
 *                                                       rule 2; a token sees itself)
 *               && q_hash[i] == k_hash[j]              (Hash-sparse only,
 *                                                       "2. Hash-Sparse" rule 3)
 *   O[i]   = sum_j softmax_j(scale * q_i . k_j over valid j) v_j
 *   lse[i] = log sum_{valid j} exp(scale * q_i . k_j)   (natural log)
 *   A row with no valid key gets O[i] = 0 and lse[i] = -inf (the page leaves
 *   this case open; this is the library's definition).
 * Tiles of `block` query rows x `block` key rows are skipped when every query
 * precedes every key ("1. QK-Sparse" rule 1) or, in Hash-sparse mode, when the
 * two blocks' bucket ranges do not overlap ("2. Hash-Sparse" rules 1-2); the
 * skipped tiles hold no valid pair, so the result is exact.  The Hash-sparse
 * entry points below also skip the tiles that pass the range test yet hold
 * no valid pair (the exact test of scfa_block_meta_exact); that changes no
 * output bit.
 *
 * Conventions shared by all entry points
 * --------------------------------------
 * Memory.  Every data pointer is DEVICE memory owned by the caller.  The
 *   library never allocates, never frees, keeps no state between calls, and is
 *   safe to call from several host threads.  Scratch memory comes from the
 *   caller's `workspace` (device memory, >= scfa_workspace_size(...) bytes,
 *   256-byte aligned); it may be reused freely between calls that are ordered
 *   on one stream.
 * Layout.  Q, K, V, O, dO, dQ, dK, dV are contiguous [B, H, T, d] (d fastest),
 *   16-byte aligned.  q_idx, q_hash, lse are contiguous [B, H, Tq]; k_idx,
 *   k_hash are [B, H, Tk]; all int32 or float32, 4-byte aligned.
 * Values.  Original positions satisfy 0 <= idx < 2147483647.  Bucket ids are
 *   any int32 (attention only compares them).  Inputs need not be sorted by
 *   position or bucket: sorting only changes speed, never the result.
 * Ragged lengths.  Heads whose kept counts differ share the [B,H,T,...]
 *   layout padded to the longest head: a padding query row carries position
 *   -1 (it admits no key: output 0, lse -inf, zero gradients) and a padding
 *   key row position 2147483647 (no query admits it; its dK, dV are 0).
 *   Blocks made only of padding are pruned like any other dead tile, so the
 *   work follows each head's own length.  Padding rows' values are ignored
 *   (keep them finite).
 * Types.  dtype SCFA_DTYPE_BF16: tensors are bfloat16, products accumulate in
 *   float32 on the matrix cores, softmax is float32, P is rounded to bf16
 *   before the P.V product, outputs are rounded once.  SCFA_DTYPE_FP32: every
 *   tensor and every operation is float32.
 * Supported sizes.  d in {64, 128}; block in {64, 128}; B, H >= 1; Tq, Tk >= 0
 *   with B*H*max(Tq,Tk)*d < 2^31; scale finite and > 0 (the usual choice is
 *   1/sqrt(d)).
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  Work is
 *   enqueued asynchronously; the call returns without synchronising and
 *   device-side faults surface at the caller's next synchronisation.
 * Errors.  Every argument is validated on the host before anything is
 *   enqueued.  On a non-zero status nothing has been enqueued and every output
 *   is untouched (except SCFA_ERR_HIP, raised by a failing launch, after
 *   which earlier kernels of the same call may have run).
 *   scfa_last_error() returns a message for the calling thread's last error.
 */
#ifndef SCFA_H
#define SCFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SCFA_OK 0
#define SCFA_ERR_INVALID_ARGUMENT 1   /* null pointer, bad size, misalignment */
#define SCFA_ERR_UNSUPPORTED 2        /* d, block, dtype or n_buckets outside the supported set */
#define SCFA_ERR_WORKSPACE_TOO_SMALL 3
#define SCFA_ERR_HIP 4                /* a HIP launch failed; see scfa_last_error() */

/* Element types. */
#define SCFA_DTYPE_BF16 0
#define SCFA_DTYPE_FP32 1

/* Flags (bitwise OR). */
#define SCFA_FLAG_NO_PRUNE (1u << 0)      /* visit every tile, masking each one; the result is
                                             bit-identical to the pruned run (test aid) */
#define SCFA_FLAG_FORCE_MASK (1u << 1)    /* apply the element mask on mask-free tiles too;
                                             bit-identical results (test aid) */
#define SCFA_FLAG_ZERO_FILL (1u << 3)     /* scfa_scatter_rows: zero every destination row
                                             first, so rows no index names read 0 */
#define SCFA_FLAG_IDX_ASCENDING (1u << 2) /* scfa_lsh_bucket_sort: the caller guarantees idx is
                                             strictly ascending within each (b, h), which lets the
                                             sort run one pass instead of five */
#define SCFA_FLAG_ORIG_ROWS (1u << 4)     /* list entry points with q_rows and k_rows: outputs (o,
                                             lse, dq, dk, dv) and the backward's o / lse inputs are
                                             indexed by the caller's rows (q_rows[i], k_rows[j]),
                                             not by the view's rows; the results equal the view-
                                             ordered ones put back with scfa_scatter_rows */

/* Operation ids for scfa_workspace_size. */
#define SCFA_OP_QK_FWD 0
#define SCFA_OP_QK_BWD 1
#define SCFA_OP_HASH_FWD 2
#define SCFA_OP_HASH_BWD 3
#define SCFA_OP_LSH_SORT 4
#define SCFA_OP_BLOCK_META_EXACT 5

/*
 * QK-sparse forward ("1. QK-Sparse": compact Q/K/V plus the original indices
 * of the kept queries and keys).
 *   q [B,H,Tq,d], k and v [B,H,Tk,d] (dtype); q_idx [B,H,Tq], k_idx [B,H,Tk].
 *   Passing q_idx == k_idx == NULL selects dense causal attention with
 *   positions 0..Tq-1 and 0..Tk-1 (the library's dense-causal baseline; it needs
 *   no workspace).  Exactly one of them NULL is an error.
 *   Outputs: o [B,H,Tq,d] (dtype), lse [B,H,Tq] float32, natural log.
 */
int scfa_qk_sparse_fwd(const void *q, const void *k, const void *v,
                       const int32_t *q_idx, const int32_t *k_idx,
                       void *o, float *lse,
                       int B, int H, int Tq, int Tk, int d, int block, float scale,
                       int dtype, unsigned flags,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * QK-sparse backward: gradients of sum(O * dout) with respect to q, k, v,
 * recomputing P from the forward's lse (no T x T state is kept).
 *   Source: the page describes no backward pass.  Its LM-training results
 *   ("实验与结果" > "QK-Sparse LM training", Fig. 8: the model that drops 30 %
 *   of queries and keys trains 1.9x faster) need one; this is the analytic
 *   gradient of the forward above: dV = P^T dO, dS = P * (dO V^T - D) with
 *   D_i = dO_i . O_i, dQ = scale dS K, dK = scale dS^T Q, over the same live
 *   tiles and element mask.
 *   o and lse must be the forward's outputs for the same inputs; dout is
 *   [B,H,Tq,d].  Outputs dq [B,H,Tq,d], dk and dv [B,H,Tk,d] (dtype), fully
 *   overwritten.  Rows with no valid key contribute nothing.
 */
int scfa_qk_sparse_bwd(const void *q, const void *k, const void *v,
                       const void *o, const float *lse, const void *dout,
                       const int32_t *q_idx, const int32_t *k_idx,
                       void *dq, void *dk, void *dv,
                       int B, int H, int Tq, int Tk, int d, int block, float scale,
                       int dtype, unsigned flags,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Hash-sparse forward ("2. Hash-Sparse": original indices plus bucket ids;
 * attention is exact within buckets).  Same as scfa_qk_sparse_fwd plus
 * q_hash [B,H,Tq] and k_hash [B,H,Tk] (required, int32).  q_idx and k_idx are
 * required here.
 */
int scfa_hash_sparse_fwd(const void *q, const void *k, const void *v,
                         const int32_t *q_idx, const int32_t *k_idx,
                         const int32_t *q_hash, const int32_t *k_hash,
                         void *o, float *lse,
                         int B, int H, int Tq, int Tk, int d, int block, float scale,
                         int dtype, unsigned flags,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Hash-sparse backward; arguments as scfa_qk_sparse_bwd plus q_hash, k_hash.
 *   Source: as for the QK-sparse backward, the page gives no backward; its
 *   Hash-sparse LM-training results ("实验与结果" > "Hash-Sparse LM training",
 *   Fig. 6: 2.0x at 8k and 3.3x at 16k tokens, and the introduction) need one.
 *   Same analytic gradient, with the Hash-sparse element mask.
 */
int scfa_hash_sparse_bwd(const void *q, const void *k, const void *v,
                         const void *o, const float *lse, const void *dout,
                         const int32_t *q_idx, const int32_t *k_idx,
                         const int32_t *q_hash, const int32_t *k_hash,
                         void *dq, void *dk, void *dv,
                         int B, int H, int Tq, int Tk, int d, int block, float scale,
                         int dtype, unsigned flags,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Hash-sparse forward that allocates nothing and takes no workspace.  For
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Arguments, results
 * and errors are those of scfa_hash_sparse_fwd; the caller still passes every
 * input and output.  Its scratch (block statistics, bucket segments, live-tile
 * lists) is a static device array of scfa_noalloc_scratch_bytes() bytes (32
 * MiB), one copy per GPU, held from the first call on that GPU until the
 * process ends.  A shape whose scratch exceeds it (scfa_workspace_size(
 * SCFA_OP_HASH_FWD, ...) > scfa_noalloc_scratch_bytes(), e.g. more than about
 * 40 heads of 16,384 tokens at block 64) is rejected with
 * SCFA_ERR_WORKSPACE_TOO_SMALL before anything touches the GPU.  Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (several
 * streams or host threads) race and give wrong results; calls ordered on one
 * stream are safe.  The array's previous contents never matter (every value is
 * written before it is read), so nothing needs clearing between calls.
 */
int scfa_hash_sparse_fwd_noalloc(const void *q, const void *k, const void *v,
                                 const int32_t *q_idx, const int32_t *k_idx,
                                 const int32_t *q_hash, const int32_t *k_hash,
                                 void *o, float *lse,
                                 int B, int H, int Tq, int Tk, int d, int block, float scale,
                                 int dtype, unsigned flags, void *stream);

/* Bytes of the static scratch array scfa_hash_sparse_fwd_noalloc uses per GPU. */
size_t scfa_noalloc_scratch_bytes(void);

/*
 * LSH bucketing and the (bucket, original position) reordering that feeds
 * Hash-sparse attention ("why dynamic sparsity breaks it": LSH groups similar
 * tokens into buckets; tokens reordered by hash keep their original positions
 * for causality).
 *   x [B,H,T,d] (dtype) in any row order; idx [B,H,T] int32 original positions
 *   of the rows (NULL = 0..T-1); R [H,d,n_buckets/2] float32, one random
 *   rotation per head shared by the batch.
 *   x_rows (nullable) [B,H,T] int32 and T_x: token t of sequence (b,h) is row
 *   x_rows[b,h,t] (clamped into [0, T_x)) of an x of T_x rows per head, e.g.
 *   the kept tokens of a full-length tensor after dropping ("1. QK-Sparse":
 *   kept tokens keep their original positions), read without compacting it.
 *   NULL: token t is row t and T_x must be 0 or T.  With x_rows, x_sorted and
 *   companion must be NULL (SCFA_ERR_UNSUPPORTED).  B*H*T*d < 2^31 always;
 *   x itself may hold up to 2^40 elements (its rows are addressed in 64 bits).
 *   bucket(x) = first index of the maximum of [x.R, -x.R], where each x.R[:,c]
 *   is accumulated in float64 in increasing coordinate order (products of a
 *   bf16/fp32 by an fp32 are exact in float64, so the result is bit-exact and
 *   reproducible).  n_buckets is even, 2 <= n_buckets <= 1024.
 *   Rows are then ordered by (bucket, idx) ascending (unique: positions are
 *   distinct within a sequence).  Outputs [B,H,T] int32:
 *     perm[s]        = source row of sorted slot s,
 *     hash_sorted[s] = bucket(x[perm[s]]),  idx_sorted[s] = idx[perm[s]].
 *   x_sorted (nullable) receives x[perm] and companion_sorted (nullable)
 *   receives companion[perm] for a second [B,H,T,d] tensor of the same dtype
 *   (e.g. V with K's order, or dO with Q's order).
 *   flags: SCFA_FLAG_IDX_ASCENDING as above (implied when idx is NULL).
 */
int scfa_lsh_bucket_sort(const void *x, const int32_t *x_rows, int T_x, const int32_t *idx, const float *R,
                         int n_buckets, int B, int H, int T, int d, int dtype, unsigned flags,
                         int32_t *hash_sorted, int32_t *idx_sorted, int32_t *perm,
                         void *x_sorted, const void *companion, void *companion_sorted,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Block metadata, exposed for inspection and bit-exact testing.  Block b of a
 * sequence covers compact rows [b*block, min((b+1)*block, T)).
 *   q_stats [B,H,nq,4], k_stats [B,H,nk,4] int32: (min idx, max idx, min hash,
 *   max hash) over the block's real rows (hash entries 0 without hashes).
 *   Tile (i,j) is live iff qmax_idx(i) >= kmin_idx(j) and, with hashes, the
 *   bucket ranges [min,max] of blocks i and j overlap ("1. QK-Sparse" rule 1,
 *   "2. Hash-Sparse" rules 1-2).  It is mask-free iff kmax_idx(j) <=
 *   qmin_idx(i) and, with hashes, both blocks hold one and the same bucket.
 *   row_count [B,H,nq]; row_list [B,H,nq,nk]: the first row_count entries of
 *   each row are the live key blocks j, ascending, each stored as
 *   j | (mask_free << 31); the rest of the row is unspecified.
 *   col_count [B,H,nk]; col_list [B,H,nk,nq]: the same per key block (query
 *   blocks i ascending).  col_count/col_list may both be NULL.
 *   q_hash and k_hash are both NULL (QK-sparse) or both non-NULL.
 */
int scfa_block_meta(const int32_t *q_idx, const int32_t *k_idx,
                    const int32_t *q_hash, const int32_t *k_hash,
                    int B, int H, int Tq, int Tk, int block,
                    int32_t *q_stats, int32_t *k_stats,
                    int32_t *row_count, int32_t *row_list,
                    int32_t *col_count, int32_t *col_list, void *stream);

/*
 * scfa_block_meta with exact tile liveness in Hash-sparse mode.  The page's
 * block rule ("2. Hash-Sparse" rules 1-2: keep the tiles whose query and key
 * buckets match, drop the acausal ones) read literally keeps a tile only when
 * one of its queries and one of its keys share a bucket in causal order, i.e.
 * when the tile holds a valid pair.  The bucket-range test of scfa_block_meta
 * also keeps tiles where every bucket the blocks share has all its keys after
 * all its queries.  Here a tile is live iff it passes the range test and some
 * bucket h present in both blocks has min k_idx over the key rows of bucket h
 * <= max q_idx over the query rows of bucket h, which is exactly "the tile
 * holds a valid pair", for any number of distinct buckets per block.
 * Mask-free flags, list layout and the other arguments are as in
 * scfa_block_meta; attention over these lists gives bit-identical results (a
 * skipped tile would only add exact zeros).  In QK-sparse mode (hashes NULL)
 * the range test is already exact and the lists equal scfa_block_meta's.
 *   workspace: device scratch of scfa_workspace_size(SCFA_OP_BLOCK_META_EXACT,
 *   B, H, Tq, Tk, 0, block, 0) bytes, 256-byte aligned (per block: one record
 *   per distinct bucket with the min and max position of its rows); unused
 *   (may be NULL) in QK-sparse mode.
 */
int scfa_block_meta_exact(const int32_t *q_idx, const int32_t *k_idx,
                          const int32_t *q_hash, const int32_t *k_hash,
                          int B, int H, int Tq, int Tk, int block,
                          int32_t *q_stats, int32_t *k_stats,
                          int32_t *row_count, int32_t *row_list,
                          int32_t *col_count, int32_t *col_list,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Attention over precomputed block lists: the single-kernel building blocks of
 * the entry points above.  A training step can build the lists once with
 * scfa_block_meta (with columns) and share them between the forward and both
 * backward kernels; each call below enqueues exactly one kernel and needs no
 * workspace.
 *   Mode: q_idx == k_idx == NULL selects dense causal (lists ignored, may be
 *   NULL); q_hash == k_hash == NULL selects QK-sparse; otherwise Hash-sparse.
 *   row_count/row_list and col_count/col_list must be scfa_block_meta's output
 *   for the same positions, buckets and block (list entries naming a block
 *   outside the sequence are skipped, never dereferenced).
 *   Row indirection (bf16 only; both NULL = none): q_rows [B,H,Tq] and k_rows
 *   [B,H,Tk] int32 make row i of the attention's Q (and of dout) row
 *   q_rows[b,h,i] of q (dout), and row j of its K and V row k_rows[b,h,j] of
 *   k and v, so a caller can attend over a reordered view (the sort
 *   permutation of scfa_lsh_bucket_sort) without copying Q, K, V and dO into
 *   that order.  Positions, buckets, lse, o (the forward's output, read by
 *   the dq call), delta and every output stay indexed by the view's rows i
 *   and j.  fp32 with row indirection is SCFA_ERR_UNSUPPORTED.
 *   Tq_src, Tk_src: rows per head of q (and dout) and of k (and v), the
 *   tensors q_rows / k_rows index; 0 means Tq / Tk.  Other values need the
 *   matching rows array: with dropped tokens ("1. QK-Sparse": the kept
 *   tokens keep their original positions) the view is the Tq kept queries
 *   and q_rows = q_idx reads them from the full-length q of Tq_src rows, so
 *   the kept rows are never copied into compact tensors.  Indices are clamped
 *   into [0, Tq_src) / [0, Tk_src) on the device (an index out of range reads
 *   a wrong row, never outside the tensor).  With SCFA_FLAG_ORIG_ROWS the
 *   outputs (and the backward's o / lse inputs) have Tq_src (dk, dv: Tk_src)
 *   rows per head; rows that no q_rows (k_rows) entry names are not written.
 *   Other arguments, layouts and flags as in scfa_*_sparse_fwd / _bwd.
 */
int scfa_attn_fwd_lists(const void *q, const void *k, const void *v,
                        const int32_t *q_idx, const int32_t *k_idx,
                        const int32_t *q_hash, const int32_t *k_hash,
                        const int32_t *q_rows, const int32_t *k_rows, int Tq_src, int Tk_src,
                        const int32_t *row_count, const int32_t *row_list,
                        void *o, float *lse,
                        int B, int H, int Tq, int Tk, int d, int block, float scale,
                        int dtype, unsigned flags, void *stream);

/* Backward, first kernel: dq [B,H,Tq,d] and the scratch `delta`,
 * [2,B,H,Tq] float32 = (rowsum(dout * o), lse * log2(e)), which the second
 * kernel reads. */
int scfa_attn_bwd_dq_lists(const void *q, const void *k, const void *v,
                           const void *o, const float *lse, const void *dout,
                           const int32_t *q_idx, const int32_t *k_idx,
                           const int32_t *q_hash, const int32_t *k_hash,
                           const int32_t *q_rows, const int32_t *k_rows, int Tq_src, int Tk_src,
                           const int32_t *row_count, const int32_t *row_list,
                           void *dq, float *delta,
                           int B, int H, int Tq, int Tk, int d, int block, float scale,
                           int dtype, unsigned flags, void *stream);

/* Backward, second kernel: dk, dv [B,H,Tk,d] from the [2,B,H,Tq] scratch
 * `delta` written by scfa_attn_bwd_dq_lists (enqueue that one first on the
 * same stream). */
int scfa_attn_bwd_dkdv_lists(const void *q, const void *k, const void *v,
                             const float *lse, const void *dout, const float *delta,
                             const int32_t *q_idx, const int32_t *k_idx,
                             const int32_t *q_hash, const int32_t *k_hash,
                             const int32_t *q_rows, const int32_t *k_rows, int Tq_src, int Tk_src,
                             const int32_t *col_count, const int32_t *col_list,
                             void *dk, void *dv,
                             int B, int H, int Tq, int Tk, int d, int block, float scale,
                             int dtype, unsigned flags, void *stream);

/*
 * Packed ragged heads ("varlen").  Dropping tokens per head leaves each head
 * its own kept count ("SCFA solution > 1. QK-Sparse": compact tensors; the
 * counts differ per head under dynamic pruning).  These calls take the heads
 * packed back to back, with no padding:
 *   q_offsets, k_offsets: [B*H + 1] int32 DEVICE arrays, non-decreasing, with
 *   offsets[0] = 0: head bh = b*H + h owns packed query rows q_offsets[bh] ..
 *   q_offsets[bh+1] - 1 (keys: k_offsets), at most max_Tq (max_Tk) of them.
 *   total_q = q_offsets[B*H], total_k = k_offsets[B*H] (passed so the host can
 *   check sizes).  Tensors: q, o, dout, dq [total_q, d]; k, v, dk, dv
 *   [total_k, d]; q_idx, q_hash, lse [total_q]; k_idx, k_hash [total_k];
 *   delta [2, total_q].  Positions and buckets are per head, as elsewhere.
 *   Lists keep the fixed-stride layout of scfa_block_meta sized by the maximum
 *   lengths: row_count [B,H,nq], row_list [B,H,nq,nk] with nq = ceil(max_Tq /
 *   block), nk = ceil(max_Tk / block); blocks past a head's length have no
 *   live tiles.  Work follows each head's own length: work groups past it exit
 *   at once.  Row indirection and the stored-dS backward are not available
 *   here (SCFA_ERR_UNSUPPORTED).  Offsets that break these rules (descending,
 *   or beyond the tensors) are not detected on the host (they live on the
 *   device); the device clamps each head's first row into [0, total] and its
 *   length into [0, min(max_T, total - first row)], so malformed offsets give
 *   wrong results but no access leaves the packed tensors.
 *   The meta call applies the exact tile rule (scfa_block_meta_exact) and takes
 *   its workspace (scfa_workspace_size(SCFA_OP_BLOCK_META_EXACT, B, H, max_Tq,
 *   max_Tk, 0, block, 0) bytes; NULL in QK-sparse mode).  Everything else is as
 *   in the fixed-length list entry points.
 */
int scfa_block_meta_varlen(const int32_t *q_offsets, const int32_t *k_offsets, int total_q, int total_k,
                           const int32_t *q_idx, const int32_t *k_idx,
                           const int32_t *q_hash, const int32_t *k_hash,
                           int B, int H, int max_Tq, int max_Tk, int block,
                           int32_t *q_stats, int32_t *k_stats,
                           int32_t *row_count, int32_t *row_list,
                           int32_t *col_count, int32_t *col_list,
                           void *workspace, size_t workspace_bytes, void *stream);
int scfa_attn_fwd_varlen(const void *q, const void *k, const void *v,
                         const int32_t *q_offsets, const int32_t *k_offsets, int total_q, int total_k,
                         const int32_t *q_idx, const int32_t *k_idx,
                         const int32_t *q_hash, const int32_t *k_hash,
                         const int32_t *row_count, const int32_t *row_list,
                         void *o, float *lse,
                         int B, int H, int max_Tq, int max_Tk, int d, int block, float scale,
                         int dtype, unsigned flags, void *stream);
int scfa_attn_bwd_dq_varlen(const void *q, const void *k, const void *v,
                            const void *o, const float *lse, const void *dout,
                            const int32_t *q_offsets, const int32_t *k_offsets, int total_q, int total_k,
                            const int32_t *q_idx, const int32_t *k_idx,
                            const int32_t *q_hash, const int32_t *k_hash,
                            const int32_t *row_count, const int32_t *row_list,
                            void *dq, float *delta,
                            int B, int H, int max_Tq, int max_Tk, int d, int block, float scale,
                            int dtype, unsigned flags, void *stream);
int scfa_attn_bwd_dkdv_varlen(const void *q, const void *k, const void *v,
                              const float *lse, const void *dout, const float *delta,
                              const int32_t *q_offsets, const int32_t *k_offsets, int total_q, int total_k,
                              const int32_t *q_idx, const int32_t *k_idx,
                              const int32_t *q_hash, const int32_t *k_hash,
                              const int32_t *col_count, const int32_t *col_list,
                              void *dk, void *dv,
                              int B, int H, int max_Tq, int max_Tk, int d, int block, float scale,
                              int dtype, unsigned flags, void *stream);

/*
 * Backward with stored dS: the dK/dV kernel keeps every live tile's dS (the
 * bf16 values its dK product uses) and dQ becomes a plain block-sparse
 * product dQ = scale * dS K over the row lists, with no exponent, mask or dP
 * recomputed.  The gradients are the analytic ones of scfa_qk_sparse_bwd /
 * scfa_hash_sparse_bwd (the page gives no backward; its LM-training results,
 * "实验与结果" > "Hash-Sparse LM training" and "QK-Sparse LM training", need
 * one).  bf16 only, pruned modes only (positions required; no
 * SCFA_FLAG_NO_PRUNE).  Order on one stream:
 *   scfa_block_meta[_exact] (with columns) -> scfa_tile_slots ->
 *   forward -> scfa_attn_bwd_prep -> scfa_attn_bwd_dkdv_ds_lists ->
 *   scfa_attn_bwd_dq_ds_lists.
 * ds: device buffer of ds_tiles tiles of block x block bf16 (tile = dS^T of
 *   one live tile, key-major: [key][query]), 16-byte aligned, caller-owned.
 *   The tiles needed are col_base[B*H*nk] (the live-tile count, on the
 *   device).  If that exceeds ds_tiles nothing is stored and dQ falls back to
 *   recomputing S, P and dP (the scfa_attn_bwd_dq_lists kernel): results stay
 *   correct, only slower.  col_base and row_slot must be scfa_tile_slots'
 *   output for the same lists; with other values the gradients are wrong, but
 *   no tile is written or read outside [0, ds_tiles).
 */

/* Slot numbering of the live tiles.  Key block c = (b*H + h)*nk + j owns
 * slots col_base[c] .. col_base[c] + col_count[c] - 1 in its column-list
 * order; col_base [B*H*nk + 1] int32 (exclusive scan of the column counts,
 * the total last).  row_slot [B,H,nq,nk] int32: entry t of query block i's
 * row list (key block j) is stored in slot row_slot[b,h,i,t] (the first
 * row_count entries of each row are written).  Lists as from scfa_block_meta. */
int scfa_tile_slots(const int32_t *row_count, const int32_t *row_list,
                    const int32_t *col_count, const int32_t *col_list,
                    int B, int H, int Tq, int Tk, int block,
                    int32_t *col_base, int32_t *row_slot, void *stream);

/* Backward preprocess: delta [2,B,H,Tq] float32 = (rowsum(dout * o),
 * lse * log2(e)), as scfa_attn_bwd_dq_lists writes it.  o and lse are the
 * forward's outputs (view rows; the caller's rows with SCFA_FLAG_ORIG_ROWS,
 * the only flag), dout [B,H,Tq_src,d] bf16, read through q_rows when non-NULL
 * (as in the list entry points; Tq_src 0 means Tq). */
int scfa_attn_bwd_prep(const void *o, const float *lse, const void *dout, const int32_t *q_rows, int Tq_src,
                       float *delta, int B, int H, int Tq, int d, int dtype, unsigned flags, void *stream);

/* dK, dV as scfa_attn_bwd_dkdv_lists (reading delta from scfa_attn_bwd_prep),
 * also writing each live tile's dS into slot col_base[...] + list position of
 * ds (when every tile fits). */
int scfa_attn_bwd_dkdv_ds_lists(const void *q, const void *k, const void *v,
                                const float *lse, const void *dout, const float *delta,
                                const int32_t *q_idx, const int32_t *k_idx,
                                const int32_t *q_hash, const int32_t *k_hash,
                                const int32_t *q_rows, const int32_t *k_rows, int Tq_src, int Tk_src,
                                const int32_t *col_count, const int32_t *col_list,
                                const int32_t *col_base, void *ds, long long ds_tiles,
                                void *dk, void *dv,
                                int B, int H, int Tq, int Tk, int d, int block, float scale,
                                int dtype, unsigned flags, void *stream);

/* dq from the stored dS tiles (enqueue after scfa_attn_bwd_dkdv_ds_lists on
 * the same stream).  The remaining arguments are those of
 * scfa_attn_bwd_dq_lists, used only by the recomputing fallback (which also
 * rewrites delta with the same values). */
int scfa_attn_bwd_dq_ds_lists(const void *q, const void *k, const void *v,
                              const void *o, const float *lse, const void *dout,
                              const int32_t *q_idx, const int32_t *k_idx,
                              const int32_t *q_hash, const int32_t *k_hash,
                              const int32_t *q_rows, const int32_t *k_rows, int Tq_src, int Tk_src,
                              const int32_t *row_count, const int32_t *row_list,
                              const int32_t *row_slot, const int32_t *col_base,
                              const void *ds, long long ds_tiles,
                              void *dq, float *delta,
                              int B, int H, int Tq, int Tk, int d, int block, float scale,
                              int dtype, unsigned flags, void *stream);

/*
 * Row gather and scatter: the steps either side of the attention path.
 * Dropping tokens compacts Q/K/V to the kept rows, and Hash-sparse attention
 * reorders tokens by bucket; every row keeps its original position ("why
 * dynamic sparsity breaks it"; "1. QK-Sparse": compact tensors plus q_idx /
 * k_idx).  These two calls build the compact or reordered inputs and put
 * outputs and gradients back at their original rows.
 *   scfa_gather_rows:  dst[b,h,i,:] = src[b,h,index[b,h,i],:]  for i < T_dst
 *     src [B,H,T_src,d], index [B,H,T_dst] int32, dst [B,H,T_dst,d].  An index
 *     outside [0, T_src) yields a zero row.  Compaction: index = kept
 *     positions (q_idx / k_idx); reordering: index = the sort's perm.
 *   scfa_scatter_rows: dst[b,h,index[b,h,i],:] = src[b,h,i,:] for i < T_src
 *     src [B,H,T_src,d], index [B,H,T_src] int32, dst [B,H,T_dst,d].  Rows
 *     whose index is outside [0, T_dst) are dropped; when two rows name the
 *     same destination, which one lands is unspecified.  flags:
 *     SCFA_FLAG_ZERO_FILL zeroes dst first (un-compaction: dropped rows 0).
 *     Un-sorting: index = perm, T_dst = T_src; un-compaction: index = q_idx.
 *   dtype as above (bf16 or fp32); d >= 1 with d * sizeof(dtype) a multiple
 *   of 16 bytes and at most 4096 bytes; B*H <= 65535; src/dst 16-byte
 *   aligned, index 4-byte aligned; src and dst must not overlap (other
 *   shapes: SCFA_ERR_UNSUPPORTED or SCFA_ERR_INVALID_ARGUMENT).  Device
 *   pointers owned by the caller; no workspace.
 */
int scfa_gather_rows(const void *src, const int32_t *index, void *dst,
                     int B, int H, int T_src, int T_dst, int d, int dtype, void *stream);
int scfa_scatter_rows(const void *src, const int32_t *index, void *dst,
                      int B, int H, int T_src, int T_dst, int d, int dtype, unsigned flags, void *stream);

/*
 * Row clear: dst[b,h,index[b,h,i],:] = 0 for i < n.  dst [B,H,T,d], index
 * [B,H,n] int32; indices outside [0, T) are skipped.  With attention that
 * reads the kept rows of full-length tensors in place and writes its outputs
 * at the kept positions (q_rows / k_rows with Tq_src / Tk_src and
 * SCFA_FLAG_ORIG_ROWS), this gives the dropped positions ("1. QK-Sparse":
 * dropped tokens take no part) their zero rows, with index = the dropped
 * positions, so no output is compacted or scattered.  dtype, d, B*H and
 * alignment limits as for scfa_gather_rows; no workspace.
 */
int scfa_zero_rows(void *dst, const int32_t *index, int B, int H, int n, int T, int d, int dtype, void *stream);

/*
 * Bytes of workspace an operation needs (0 for invalid arguments).  For the
 * attention ops and SCFA_OP_BLOCK_META_EXACT d and n_buckets are ignored; for
 * SCFA_OP_LSH_SORT Tq is the sequence length T and Tk, d, block are ignored.  The size is an upper
 * bound valid for every flag combination.
 */
size_t scfa_workspace_size(int op, int B, int H, int Tq, int Tk, int d, int block, int n_buckets);

/* Message for the calling thread's most recent non-zero status ("" if none). */
const char *scfa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SCFA_H */
