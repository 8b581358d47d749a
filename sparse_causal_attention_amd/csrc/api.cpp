// C ABI of the SCFA library: argument validation, workspace carving and
// dispatch to the kernel launchers.  Nothing is enqueued unless every
// argument is valid; the library never allocates device memory.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/scfa.h"
#include "scfa_internal.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return SCFA_OK;
}

int hip_fail(hipError_t e, const char *where) {
  return fail(SCFA_ERR_HIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

constexpr size_t kAlign = scfa::kWsAlign;
size_t round_up(size_t x) { return scfa::ws_round(x); }
int nblocks(int T, int block) { return (T + block - 1) / block; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Pointer that must be non-null when `elems` > 0 and aligned to `al` bytes.
int check_ptr(const void *p, long long elems, size_t al, const char *name) {
  if (elems <= 0) return SCFA_OK;
  if (p == nullptr) return fail(SCFA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned(p, al)) return fail(SCFA_ERR_INVALID_ARGUMENT, "%s is not %zu-byte aligned", name, al);
  return SCFA_OK;
}

struct Shape {
  int B, H, Tq, Tk, d, block, dtype;
  float scale;
};

int check_shape(const Shape &s) {
  if (s.B < 1 || s.H < 1) return fail(SCFA_ERR_INVALID_ARGUMENT, "B and H must be >= 1 (got %d, %d)", s.B, s.H);
  if (s.Tq < 0 || s.Tk < 0) return fail(SCFA_ERR_INVALID_ARGUMENT, "Tq and Tk must be >= 0 (got %d, %d)", s.Tq, s.Tk);
  if (s.d != 64 && s.d != 128) return fail(SCFA_ERR_UNSUPPORTED, "head dim d=%d unsupported (64 or 128)", s.d);
  if (s.block != 64 && s.block != 128) return fail(SCFA_ERR_UNSUPPORTED, "block=%d unsupported (64 or 128)", s.block);
  if (s.dtype != SCFA_DTYPE_BF16 && s.dtype != SCFA_DTYPE_FP32)
    return fail(SCFA_ERR_UNSUPPORTED, "dtype=%d unsupported", s.dtype);
  if (!(std::isfinite(s.scale) && s.scale > 0.f)) return fail(SCFA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
  const long long T = s.Tq > s.Tk ? s.Tq : s.Tk;
  if ((long long)s.B * s.H * T * s.d >= (1ll << 31))
    return fail(SCFA_ERR_INVALID_ARGUMENT, "B*H*max(Tq,Tk)*d must be < 2^31");
  return SCFA_OK;
}

size_t attn_ws(bool bwd, int B, int H, int Tq, int Tk, int block) {
  const size_t BH = (size_t)B * H;
  const size_t nq = nblocks(Tq, block), nk = nblocks(Tk, block);
  size_t n = round_up(BH * nq * 16) + round_up(BH * nk * 16) + round_up(BH * nq * 4) + round_up(BH * nq * nk * 4) +
             scfa::meta_seg_bytes(BH, nq, nk, block);
  if (bwd) n += round_up(BH * nk * 4) + round_up(BH * nk * nq * 4) + round_up(2 * BH * (size_t)Tq * 4);
  return n;
}

struct Carver {
  char *p;
  template <typename T>
  T *take(size_t bytes) {
    T *r = reinterpret_cast<T *>(p);
    p += round_up(bytes);
    return r;
  }
};

int check_ws(void *ws, size_t have, size_t need) {
  if (need == 0) return SCFA_OK;
  if (ws == nullptr) return fail(SCFA_ERR_INVALID_ARGUMENT, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned(ws, kAlign)) return fail(SCFA_ERR_INVALID_ARGUMENT, "workspace is not %zu-byte aligned", kAlign);
  if (have < need) return fail(SCFA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, %zu needed", have, need);
  return SCFA_OK;
}

enum Kind { kFwd, kBwdAll, kBwdDq, kBwdDkdv };
enum Api { kApiQK, kApiHash, kApiLists };

// Everything an attention entry point receives.
struct AttnCall {
  Kind kind;
  Api api;
  const void *q, *k, *v, *o;
  const float *lse;
  const void *dout;
  const int32_t *q_idx, *k_idx, *q_hash, *k_hash;
  const int32_t *row_cnt, *row_list, *col_cnt, *col_list;  // list entry points only
  const int32_t *q_rows, *k_rows;                          // list entry points only (nullable)
  int Tq_src, Tk_src;  // rows per head of q / dout and of k / v (list entry points; 0 = Tq, Tk)
  void *out_o;
  float *out_lse;
  void *dq, *dk, *dv;
  float *delta;  // list entry points only
  // stored-dS backward (list entry points): the dS buffer and the tile slots
  bool ds_path;
  void *ds;
  long long ds_tiles;
  const int32_t *row_slot, *col_base;
  // packed ragged heads (varlen entry points): offsets [BH+1] and packed row counts; Shape's Tq, Tk
  // are then the maximum head lengths
  const int32_t *q_off, *k_off;
  long long total_q, total_k;
  Shape s;
  unsigned flags;
  void *ws;
  size_t ws_bytes;
  void *stream;
};

// Shared implementation of every attention entry point.
int attention(const AttnCall &c) {
  const Shape &s = c.s;
  int rc = check_shape(s);
  if (rc) return rc;
  const unsigned known = SCFA_FLAG_NO_PRUNE | SCFA_FLAG_FORCE_MASK | (c.api == kApiLists ? SCFA_FLAG_ORIG_ROWS : 0u);
  if (c.flags & ~known) return fail(SCFA_ERR_INVALID_ARGUMENT, "unknown flags 0x%x", c.flags);
  const long long BH = (long long)s.B * s.H;
  const bool varlen = c.q_off != nullptr || c.k_off != nullptr;
  if (varlen) {
    if (c.q_off == nullptr || c.k_off == nullptr)
      return fail(SCFA_ERR_INVALID_ARGUMENT, "q_offsets and k_offsets must both be set");
    if (!aligned(c.q_off, 4) || !aligned(c.k_off, 4)) return fail(SCFA_ERR_INVALID_ARGUMENT, "offsets not 4-byte aligned");
    if (c.total_q < 0 || c.total_k < 0 || c.total_q * s.d >= (1ll << 31) || c.total_k * s.d >= (1ll << 31))
      return fail(SCFA_ERR_INVALID_ARGUMENT, "packed row counts must be >= 0 and rows*d < 2^31");
    if (c.q_rows || c.k_rows || c.ds_path) return fail(SCFA_ERR_UNSUPPORTED, "ragged heads: no row indirection or stored dS");
  }
  // Rows per head of the caller's tensors: the view's Tq, Tk unless row indirection reads tensors of
  // another length (q / dout: Tqs, k / v: Tks); the outputs follow them with SCFA_FLAG_ORIG_ROWS.
  const bool orig_rows = (c.flags & SCFA_FLAG_ORIG_ROWS) != 0;
  const int Tqs = c.Tq_src > 0 ? c.Tq_src : s.Tq, Tks = c.Tk_src > 0 ? c.Tk_src : s.Tk;
  if (c.Tq_src < 0 || c.Tk_src < 0) return fail(SCFA_ERR_INVALID_ARGUMENT, "Tq_src and Tk_src must be >= 0");
  if ((c.q_rows == nullptr && Tqs != s.Tq) || (c.k_rows == nullptr && Tks != s.Tk))
    return fail(SCFA_ERR_INVALID_ARGUMENT, "Tq_src / Tk_src other than Tq / Tk need q_rows / k_rows");
  if ((long long)s.B * s.H * (Tqs > Tks ? Tqs : Tks) * s.d >= (1ll << 31))
    return fail(SCFA_ERR_INVALID_ARGUMENT, "B*H*max(Tq_src,Tk_src)*d must be < 2^31");
  const int Tqo = orig_rows ? Tqs : s.Tq, Tko = orig_rows ? Tks : s.Tk;
  const long long rowsQ = varlen ? c.total_q : BH * s.Tq, rowsK = varlen ? c.total_k : BH * s.Tk;
  const long long nQi = rowsQ, nKi = rowsK;
  // element counts of the caller's inputs (s) and of the outputs (o)
  const long long nQs = (varlen ? c.total_q : BH * Tqs) * s.d, nKs = (varlen ? c.total_k : BH * Tks) * s.d;
  const long long nQoi = varlen ? c.total_q : BH * Tqo, nKo = (varlen ? c.total_k : BH * Tko) * s.d;
  const long long nQo = nQoi * s.d;
  const int nq = nblocks(s.Tq, s.block), nk = nblocks(s.Tk, s.block);
  if ((rc = check_ptr(c.q, nQs, 16, "q")) || (rc = check_ptr(c.k, nKs, 16, "k")) || (rc = check_ptr(c.v, nKs, 16, "v")))
    return rc;
  // Positions and buckets.  A pointer may be NULL when its tensor is empty
  // (T == 0): torch hands out NULL for empty tensors.
  bool dense, hashed;
  if (c.api == kApiHash) {
    dense = false;
    hashed = true;
  } else {
    dense = c.q_idx == nullptr && c.k_idx == nullptr;
    hashed = c.api == kApiLists && (c.q_hash != nullptr || c.k_hash != nullptr);
    if (hashed && dense && (nQi > 0 || nKi > 0))
      return fail(SCFA_ERR_INVALID_ARGUMENT, "bucket ids need positions (q_idx, k_idx)");
  }
  if (!dense && ((rc = check_ptr(c.q_idx, nQi, 4, "q_idx")) || (rc = check_ptr(c.k_idx, nKi, 4, "k_idx"))))
    return rc;
  if (hashed && ((rc = check_ptr(c.q_hash, nQi, 4, "q_hash")) || (rc = check_ptr(c.k_hash, nKi, 4, "k_hash"))))
    return rc;
  // tensors of each kind
  switch (c.kind) {
    case kFwd:
      if ((rc = check_ptr(c.out_o, nQo, 16, "o")) || (rc = check_ptr(c.out_lse, nQoi, 4, "lse"))) return rc;
      break;
    case kBwdAll:
    case kBwdDq:
      if ((rc = check_ptr(c.o, nQo, 16, "o")) || (rc = check_ptr(c.lse, nQoi, 4, "lse")) ||
          (rc = check_ptr(c.dout, nQs, 16, "dout")) || (rc = check_ptr(c.dq, nQo, 16, "dq")))
        return rc;
      if (c.kind == kBwdAll && ((rc = check_ptr(c.dk, nKo, 16, "dk")) || (rc = check_ptr(c.dv, nKo, 16, "dv"))))
        return rc;
      if (c.kind == kBwdDq && (rc = check_ptr(c.delta, 2 * nQi, 4, "delta"))) return rc;
      break;
    case kBwdDkdv:
      if ((rc = check_ptr(c.lse, nQoi, 4, "lse")) || (rc = check_ptr(c.dout, nQs, 16, "dout")) ||
          (rc = check_ptr(c.delta, 2 * nQi, 4, "delta")) || (rc = check_ptr(c.dk, nKo, 16, "dk")) ||
          (rc = check_ptr(c.dv, nKo, 16, "dv")))
        return rc;
      break;
  }
  if (c.q_rows || c.k_rows) {
    if (s.dtype != SCFA_DTYPE_BF16)
      return fail(SCFA_ERR_UNSUPPORTED, "q_rows / k_rows (row indirection) need dtype bf16");
    if ((rc = check_ptr(c.q_rows, c.q_rows ? nQi : 0, 4, "q_rows")) ||
        (rc = check_ptr(c.k_rows, c.k_rows ? nKi : 0, 4, "k_rows")))
      return rc;
  }
  const bool no_prune = (c.flags & SCFA_FLAG_NO_PRUNE) != 0;
  if (orig_rows && (c.q_rows == nullptr || c.k_rows == nullptr) && (nQi > 0 || nKi > 0))
    return fail(SCFA_ERR_INVALID_ARGUMENT, "SCFA_FLAG_ORIG_ROWS needs both q_rows and k_rows");
  if (c.ds_path) {
    if (s.dtype != SCFA_DTYPE_BF16) return fail(SCFA_ERR_UNSUPPORTED, "stored-dS backward needs dtype bf16");
    if (dense) return fail(SCFA_ERR_UNSUPPORTED, "stored-dS backward needs positions (pruned modes; no lists in dense)");
    if (no_prune) return fail(SCFA_ERR_UNSUPPORTED, "stored-dS backward walks the lists: SCFA_FLAG_NO_PRUNE unsupported");
    if (c.ds_tiles < 0) return fail(SCFA_ERR_INVALID_ARGUMENT, "ds_tiles must be >= 0");
    if ((rc = check_ptr(c.ds, c.ds_tiles * s.block * s.block, 16, "ds")) ||
        (rc = check_ptr(c.col_base, BH * nk + 1, 4, "col_base")))
      return rc;
    if (c.kind == kBwdDq && (rc = check_ptr(c.row_slot, BH * nq * nk, 4, "row_slot"))) return rc;
  }
  // lists (list entry points) or workspace (the others)
  if (c.api == kApiLists) {
    if (!dense && !no_prune) {
      if (c.kind != kBwdDkdv && ((rc = check_ptr(c.row_cnt, BH * nq, 4, "row_count")) ||
                                 (rc = check_ptr(c.row_list, BH * nq * nk, 4, "row_list"))))
        return rc;
      if (c.kind == kBwdDkdv && ((rc = check_ptr(c.col_cnt, BH * nk, 4, "col_count")) ||
                                 (rc = check_ptr(c.col_list, BH * nk * nq, 4, "col_list"))))
        return rc;
    }
  } else {
    const bool bwd = c.kind != kFwd;
    size_t need = attn_ws(bwd, s.B, s.H, s.Tq, s.Tk, s.block);
    if (dense) need = bwd ? round_up(2 * (size_t)BH * s.Tq * 4) : 0;
    if ((rc = check_ws(c.ws, c.ws_bytes, need))) return rc;
  }

  hipStream_t st = static_cast<hipStream_t>(c.stream);
  scfa::AttnArgs a{};
  a.q = c.q;
  a.k = c.k;
  a.v = c.v;
  a.o = c.o;
  a.dout = c.dout;
  a.lse = c.lse;
  a.out_o = c.out_o;
  a.out_lse = c.out_lse;
  a.dq = c.dq;
  a.dk = c.dk;
  a.dv = c.dv;
  a.q_idx = c.q_idx;
  a.k_idx = c.k_idx;
  a.q_hash = hashed ? c.q_hash : nullptr;
  a.k_hash = hashed ? c.k_hash : nullptr;
  a.q_rows = c.q_rows;
  a.k_rows = c.k_rows;
  a.BH = (int)BH;
  a.Tq = s.Tq;
  a.Tk = s.Tk;
  a.Tqs = Tqs;
  a.Tks = Tks;
  a.Tqo = Tqo;
  a.Tko = Tko;
  a.nq = nq;
  a.nk = nk;
  a.d = s.d;
  a.block = s.block;
  a.scale = s.scale;
  a.no_prune = no_prune ? 1 : 0;
  a.force_mask = (c.flags & SCFA_FLAG_FORCE_MASK) ? 1 : 0;
  a.orig_rows = orig_rows ? 1 : 0;
  a.q_off = c.q_off;
  a.k_off = c.k_off;
  a.q_total = c.total_q;
  a.k_total = c.total_k;
  a.delta_half = rowsQ;
  a.ds = c.ds;
  a.ds_tiles = c.ds_tiles;
  a.row_slot = c.row_slot;
  a.col_base = c.col_base;

  if (c.api == kApiLists) {
    a.row_cnt = c.row_cnt;
    a.row_list = c.row_list;
    a.col_cnt = c.col_cnt;
    a.col_list = c.col_list;
    a.delta = c.delta;
  } else {
    Carver cv{static_cast<char *>(c.ws)};
    const bool bwd = c.kind != kFwd;
    if (!dense) {
      scfa::MetaArgs m{};
      m.q_idx = c.q_idx;
      m.k_idx = c.k_idx;
      m.q_hash = a.q_hash;
      m.k_hash = a.k_hash;
      m.q_stats = cv.take<int32_t>((size_t)BH * nq * 16);
      m.k_stats = cv.take<int32_t>((size_t)BH * nk * 16);
      m.row_cnt = cv.take<int32_t>((size_t)BH * nq * 4);
      m.row_list = cv.take<int32_t>((size_t)BH * nq * nk * 4);
      int32_t *qsg = cv.take<int32_t>((size_t)BH * nq * s.block * 16);
      int32_t *ksg = cv.take<int32_t>((size_t)BH * nk * s.block * 16);
      int32_t *qns = cv.take<int32_t>((size_t)BH * nq * 4);
      int32_t *kns = cv.take<int32_t>((size_t)BH * nk * 4);
      if (hashed) m.q_segs = qsg, m.k_segs = ksg, m.q_nseg = qns, m.k_nseg = kns;  // exact tile test
      if (bwd) {
        m.col_cnt = cv.take<int32_t>((size_t)BH * nk * 4);
        m.col_list = cv.take<int32_t>((size_t)BH * nk * nq * 4);
      }
      m.BH = (int)BH;
      m.Tq = s.Tq;
      m.Tk = s.Tk;
      m.nq = nq;
      m.nk = nk;
      m.block = s.block;
      a.row_cnt = m.row_cnt;
      a.row_list = m.row_list;
      a.col_cnt = m.col_cnt;
      a.col_list = m.col_list;
      if (!no_prune) {
        hipError_t e = scfa::launch_block_meta(m, bwd, st);
        if (e != hipSuccess) return hip_fail(e, "block metadata");
      }
    }
    if (bwd) a.delta = cv.take<float>(2 * (size_t)BH * s.Tq * 4);
  }

  const int mode = hashed ? scfa::kHash : (dense ? scfa::kDense : scfa::kQK);
  const bool bf16 = s.dtype == SCFA_DTYPE_BF16;
  hipError_t e;
  if (c.kind == kFwd) {
    e = bf16 ? scfa::launch_attn_fwd_bf16(a, mode, st) : scfa::launch_attn_fwd_f32(a, mode, st);
  } else if (c.ds_path) {
    e = scfa::launch_attn_bwd_ds_bf16(a, mode, c.kind == kBwdDq ? 1 : 2, st);
  } else {
    const int part = c.kind == kBwdAll ? 3 : (c.kind == kBwdDq ? 1 : 2);
    e = bf16 ? scfa::launch_attn_bwd_bf16(a, mode, part, st) : scfa::launch_attn_bwd_f32(a, mode, part, st);
  }
  if (e != hipSuccess) return hip_fail(e, c.kind == kFwd ? "attention forward" : "attention backward");
  return ok();
}

size_t lsh_ws(int B, int H, int T, int d, int nb) {
  const size_t BH = (size_t)B * H;
  const size_t nbins = (size_t)scfa::sort_bins(nb, true);
  return round_up(BH * T * 4) + round_up(BH * nbins * scfa::sort_chunks(T) * 4) + 4 * round_up(BH * T * 4) +
         round_up((size_t)H * d * scfa::lsh_r64_cols(nb) * 8) + round_up(scfa::lsh_frag_bytes(H, d, nb)) +
         round_up((size_t)H * (nb / 2) * 4) + round_up(4) + round_up(2 * BH * nbins * 4);
}

int meta_call(const int32_t *q_idx, const int32_t *k_idx, const int32_t *q_hash, const int32_t *k_hash, int B, int H,
              int Tq, int Tk, int block, int32_t *q_stats, int32_t *k_stats, bool exact, int32_t *row_count,
              int32_t *row_list, int32_t *col_count, int32_t *col_list, void *ws, size_t ws_bytes, void *stream,
              const int32_t *q_off = nullptr, const int32_t *k_off = nullptr, long long total_q = 0,
              long long total_k = 0) {
  if (B < 1 || H < 1 || Tq < 0 || Tk < 0) return fail(SCFA_ERR_INVALID_ARGUMENT, "B, H >= 1 and Tq, Tk >= 0 required");
  if (block != 64 && block != 128) return fail(SCFA_ERR_UNSUPPORTED, "block=%d unsupported (64 or 128)", block);
  if ((q_hash == nullptr) != (k_hash == nullptr))
    return fail(SCFA_ERR_INVALID_ARGUMENT, "q_hash and k_hash must both be NULL or both set");
  if ((col_count == nullptr) != (col_list == nullptr))
    return fail(SCFA_ERR_INVALID_ARGUMENT, "col_count and col_list must both be NULL or both set");
  const long long BH = (long long)B * H;
  const long long nq = nblocks(Tq, block), nk = nblocks(Tk, block);
  if (BH * nq * nk >= (1ll << 31) || BH * (Tq > Tk ? Tq : Tk) >= (1ll << 31))
    return fail(SCFA_ERR_INVALID_ARGUMENT, "metadata too large");
  const bool varlen = q_off != nullptr || k_off != nullptr;
  if (varlen && (q_off == nullptr || k_off == nullptr || total_q < 0 || total_k < 0 || !aligned(q_off, 4) ||
                 !aligned(k_off, 4)))
    return fail(SCFA_ERR_INVALID_ARGUMENT, "ragged heads need both 4-byte aligned offsets and packed row counts >= 0");
  const long long rowsQ = varlen ? total_q : BH * Tq, rowsK = varlen ? total_k : BH * Tk;
  int rc;
  if ((rc = check_ptr(q_idx, rowsQ, 4, "q_idx")) || (rc = check_ptr(k_idx, rowsK, 4, "k_idx")) ||
      (rc = check_ptr(q_hash, q_hash ? rowsQ : 0, 4, "q_hash")) ||
      (rc = check_ptr(k_hash, k_hash ? rowsK : 0, 4, "k_hash")) ||
      (rc = check_ptr(q_stats, BH * nq * 4, 16, "q_stats")) || (rc = check_ptr(k_stats, BH * nk * 4, 16, "k_stats")) ||
      (rc = check_ptr(row_count, BH * nq, 4, "row_count")) || (rc = check_ptr(row_list, BH * nq * nk, 4, "row_list")))
    return rc;
  if (col_count && ((rc = check_ptr(col_count, BH * nk, 4, "col_count")) ||
                    (rc = check_ptr(col_list, BH * nk * nq, 4, "col_list"))))
    return rc;
  const bool use_segs = exact && q_hash != nullptr;  // QK-sparse: the range test is already exact
  if (use_segs && (rc = check_ws(ws, ws_bytes, scfa::meta_seg_bytes(BH, nq, nk, block)))) return rc;
  scfa::MetaArgs m{};
  m.q_idx = q_idx;
  m.k_idx = k_idx;
  m.q_hash = q_hash;
  m.k_hash = k_hash;
  m.q_off = q_off;
  m.k_off = k_off;
  m.q_total = total_q;
  m.k_total = total_k;
  m.q_stats = q_stats;
  m.k_stats = k_stats;
  if (use_segs) {
    Carver cv{static_cast<char *>(ws)};
    m.q_segs = cv.take<int32_t>((size_t)BH * nq * block * 16);
    m.k_segs = cv.take<int32_t>((size_t)BH * nk * block * 16);
    m.q_nseg = cv.take<int32_t>((size_t)BH * nq * 4);
    m.k_nseg = cv.take<int32_t>((size_t)BH * nk * 4);
  }
  m.row_cnt = row_count;
  m.row_list = row_list;
  m.col_cnt = col_count;
  m.col_list = col_list;
  m.BH = (int)BH;
  m.Tq = Tq;
  m.Tk = Tk;
  m.nq = (int)nq;
  m.nk = (int)nk;
  m.block = block;
  hipError_t e = scfa::launch_block_meta(m, col_count != nullptr, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "block metadata");
  return ok();
}

int rows_call(bool gather, const void *src, const int32_t *index, void *dst, int B, int H, int Ts, int Td, int d,
              int dtype, unsigned flags, void *stream) {
  if (B < 1 || H < 1 || Ts < 0 || Td < 0 || d < 1)
    return fail(SCFA_ERR_INVALID_ARGUMENT, "B, H, d >= 1 and T_src, T_dst >= 0 required");
  if (dtype != SCFA_DTYPE_BF16 && dtype != SCFA_DTYPE_FP32) return fail(SCFA_ERR_UNSUPPORTED, "dtype=%d unsupported", dtype);
  const int esize = dtype == SCFA_DTYPE_BF16 ? 2 : 4;
  if ((d * esize) % 16 != 0) return fail(SCFA_ERR_UNSUPPORTED, "row of %d bytes is not a multiple of 16", d * esize);
  if (d * esize > 4096) return fail(SCFA_ERR_UNSUPPORTED, "row of %d bytes exceeds 4096", d * esize);
  if ((long long)B * H > 65535) return fail(SCFA_ERR_UNSUPPORTED, "B*H = %lld exceeds 65535", (long long)B * H);
  if (flags & ~(gather ? 0u : SCFA_FLAG_ZERO_FILL)) return fail(SCFA_ERR_INVALID_ARGUMENT, "unknown flags 0x%x", flags);
  const long long BH = (long long)B * H;
  const long long T = Ts > Td ? Ts : Td;
  if (BH * T >= (1ll << 31) || BH * T * d >= (1ll << 40)) return fail(SCFA_ERR_INVALID_ARGUMENT, "tensors too large");
  int rc;
  const long long n_index = BH * (gather ? Td : Ts);
  if ((rc = check_ptr(src, BH * Ts * d, 16, "src")) || (rc = check_ptr(dst, BH * Td * d, 16, "dst")) ||
      (rc = check_ptr(index, n_index, 4, "index")))
    return rc;
  const char *s0 = static_cast<const char *>(src), *d0 = static_cast<const char *>(dst);
  if (BH * Ts * d > 0 && BH * Td * d > 0 && s0 < d0 + BH * Td * d * esize && d0 < s0 + BH * Ts * d * esize)
    return fail(SCFA_ERR_INVALID_ARGUMENT, "src and dst overlap");
  scfa::RowArgs r{src, index, dst, (int)BH, Ts, Td, d * esize / 16};
  const hipError_t e = gather ? scfa::launch_gather_rows(r, static_cast<hipStream_t>(stream))
                              : scfa::launch_scatter_rows(r, (flags & SCFA_FLAG_ZERO_FILL) != 0,
                                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, gather ? "gather rows" : "scatter rows");
  return ok();
}
}  // namespace

int scfa::report_error(int code, const char *msg) { return fail(code, "%s", msg); }

extern "C" {

int scfa_qk_sparse_fwd(const void *q, const void *k, const void *v, const int32_t *q_idx, const int32_t *k_idx,
                       void *o, float *lse, int B, int H, int Tq, int Tk, int d, int block, float scale, int dtype,
                       unsigned flags, void *workspace, size_t workspace_bytes, void *stream) {
  AttnCall c{};
  c.kind = kFwd;
  c.api = kApiQK;
  c.q = q, c.k = k, c.v = v, c.q_idx = q_idx, c.k_idx = k_idx, c.out_o = o, c.out_lse = lse;
  c.s = Shape{B, H, Tq, Tk, d, block, dtype, scale};
  c.flags = flags, c.ws = workspace, c.ws_bytes = workspace_bytes, c.stream = stream;
  return attention(c);
}

int scfa_qk_sparse_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                       const void *dout, const int32_t *q_idx, const int32_t *k_idx, void *dq, void *dk, void *dv,
                       int B, int H, int Tq, int Tk, int d, int block, float scale, int dtype, unsigned flags,
                       void *workspace, size_t workspace_bytes, void *stream) {
  AttnCall c{};
  c.kind = kBwdAll;
  c.api = kApiQK;
  c.q = q, c.k = k, c.v = v, c.o = o, c.lse = lse, c.dout = dout, c.q_idx = q_idx, c.k_idx = k_idx;
  c.dq = dq, c.dk = dk, c.dv = dv;
  c.s = Shape{B, H, Tq, Tk, d, block, dtype, scale};
  c.flags = flags, c.ws = workspace, c.ws_bytes = workspace_bytes, c.stream = stream;
  return attention(c);
}

int scfa_hash_sparse_fwd(const void *q, const void *k, const void *v, const int32_t *q_idx, const int32_t *k_idx,
                         const int32_t *q_hash, const int32_t *k_hash, void *o, float *lse, int B, int H, int Tq,
                         int Tk, int d, int block, float scale, int dtype, unsigned flags, void *workspace,
                         size_t workspace_bytes, void *stream) {
  AttnCall c{};
  c.kind = kFwd;
  c.api = kApiHash;
  c.q = q, c.k = k, c.v = v, c.q_idx = q_idx, c.k_idx = k_idx, c.q_hash = q_hash, c.k_hash = k_hash;
  c.out_o = o, c.out_lse = lse;
  c.s = Shape{B, H, Tq, Tk, d, block, dtype, scale};
  c.flags = flags, c.ws = workspace, c.ws_bytes = workspace_bytes, c.stream = stream;
  return attention(c);
}

int scfa_hash_sparse_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                         const void *dout, const int32_t *q_idx, const int32_t *k_idx, const int32_t *q_hash,
                         const int32_t *k_hash, void *dq, void *dk, void *dv, int B, int H, int Tq, int Tk, int d,
                         int block, float scale, int dtype, unsigned flags, void *workspace, size_t workspace_bytes,
                         void *stream) {
  AttnCall c{};
  c.kind = kBwdAll;
  c.api = kApiHash;
  c.q = q, c.k = k, c.v = v, c.o = o, c.lse = lse, c.dout = dout;
  c.q_idx = q_idx, c.k_idx = k_idx, c.q_hash = q_hash, c.k_hash = k_hash;
  c.dq = dq, c.dk = dk, c.dv = dv;
  c.s = Shape{B, H, Tq, Tk, d, block, dtype, scale};
  c.flags = flags, c.ws = workspace, c.ws_bytes = workspace_bytes, c.stream = stream;
  return attention(c);
}

int scfa_attn_fwd_lists(const void *q, const void *k, const void *v, const int32_t *q_idx, const int32_t *k_idx,
                        const int32_t *q_hash, const int32_t *k_hash, const int32_t *q_rows, const int32_t *k_rows, int Tq_src, int Tk_src,
                        const int32_t *row_count, const int32_t *row_list, void *o, float *lse, int B, int H, int Tq,
                        int Tk, int d, int block, float scale, int dtype, unsigned flags, void *stream) {
  AttnCall c{};
  c.kind = kFwd;
  c.api = kApiLists;
  c.q = q, c.k = k, c.v = v, c.q_idx = q_idx, c.k_idx = k_idx, c.q_hash = q_hash, c.k_hash = k_hash;
  c.q_rows = q_rows, c.k_rows = k_rows, c.Tq_src = Tq_src, c.Tk_src = Tk_src;
  c.row_cnt = row_count, c.row_list = row_list, c.out_o = o, c.out_lse = lse;
  c.s = Shape{B, H, Tq, Tk, d, block, dtype, scale};
  c.flags = flags, c.stream = stream;
  return attention(c);
}

int scfa_attn_bwd_dq_lists(const void *q, const void *k, const void *v, const void *o, const float *lse,
                           const void *dout, const int32_t *q_idx, const int32_t *k_idx, const int32_t *q_hash,
                           const int32_t *k_hash, const int32_t *q_rows, const int32_t *k_rows, int Tq_src, int Tk_src,
                           const int32_t *row_count, const int32_t *row_list, void *dq, float *delta, int B, int H,
                           int Tq, int Tk, int d, int block, float scale, int dtype, unsigned flags, void *stream) {
  AttnCall c{};
  c.kind = kBwdDq;
  c.api = kApiLists;
  c.q = q, c.k = k, c.v = v, c.o = o, c.lse = lse, c.dout = dout;
  c.q_idx = q_idx, c.k_idx = k_idx, c.q_hash = q_hash, c.k_hash = k_hash;
  c.q_rows = q_rows, c.k_rows = k_rows, c.Tq_src = Tq_src, c.Tk_src = Tk_src;
  c.row_cnt = row_count, c.row_list = row_list, c.dq = dq, c.delta = delta;
  c.s = Shape{B, H, Tq, Tk, d, block, dtype, scale};
  c.flags = flags, c.stream = stream;
  return attention(c);
}

int scfa_attn_bwd_dkdv_lists(const void *q, const void *k, const void *v, const float *lse, const void *dout,
                             const float *delta, const int32_t *q_idx, const int32_t *k_idx, const int32_t *q_hash,
                             const int32_t *k_hash, const int32_t *q_rows, const int32_t *k_rows, int Tq_src, int Tk_src,
                             const int32_t *col_count, const int32_t *col_list, void *dk, void *dv, int B, int H,
                             int Tq, int Tk, int d, int block, float scale, int dtype, unsigned flags, void *stream) {
  AttnCall c{};
  c.kind = kBwdDkdv;
  c.api = kApiLists;
  c.q = q, c.k = k, c.v = v, c.lse = lse, c.dout = dout, c.delta = const_cast<float *>(delta);
  c.q_idx = q_idx, c.k_idx = k_idx, c.q_hash = q_hash, c.k_hash = k_hash;
  c.q_rows = q_rows, c.k_rows = k_rows, c.Tq_src = Tq_src, c.Tk_src = Tk_src;
  c.col_cnt = col_count, c.col_list = col_list, c.dk = dk, c.dv = dv;
  c.s = Shape{B, H, Tq, Tk, d, block, dtype, scale};
  c.flags = flags, c.stream = stream;
  return attention(c);
}

int scfa_block_meta_varlen(const int32_t *q_offsets, const int32_t *k_offsets, int total_q, int total_k,
                           const int32_t *q_idx, const int32_t *k_idx, const int32_t *q_hash, const int32_t *k_hash,
                           int B, int H, int max_Tq, int max_Tk, int block, int32_t *q_stats, int32_t *k_stats,
                           int32_t *row_count, int32_t *row_list, int32_t *col_count, int32_t *col_list,
                           void *workspace, size_t workspace_bytes, void *stream) {
  if (q_offsets == nullptr || k_offsets == nullptr)
    return fail(SCFA_ERR_INVALID_ARGUMENT, "q_offsets and k_offsets are required");
  return meta_call(q_idx, k_idx, q_hash, k_hash, B, H, max_Tq, max_Tk, block, q_stats, k_stats, true, row_count,
                   row_list, col_count, col_list, workspace, workspace_bytes, stream, q_offsets, k_offsets, total_q,
                   total_k);
}

int scfa_attn_fwd_varlen(const void *q, const void *k, const void *v, const int32_t *q_offsets,
                         const int32_t *k_offsets, int total_q, int total_k, const int32_t *q_idx,
                         const int32_t *k_idx, const int32_t *q_hash, const int32_t *k_hash, const int32_t *row_count,
                         const int32_t *row_list, void *o, float *lse, int B, int H, int max_Tq, int max_Tk, int d,
                         int block, float scale, int dtype, unsigned flags, void *stream) {
  if (q_offsets == nullptr || k_offsets == nullptr)
    return fail(SCFA_ERR_INVALID_ARGUMENT, "q_offsets and k_offsets are required");
  AttnCall c{};
  c.kind = kFwd;
  c.api = kApiLists;
  c.q = q, c.k = k, c.v = v, c.q_idx = q_idx, c.k_idx = k_idx, c.q_hash = q_hash, c.k_hash = k_hash;
  c.row_cnt = row_count, c.row_list = row_list, c.out_o = o, c.out_lse = lse;
  c.q_off = q_offsets, c.k_off = k_offsets, c.total_q = total_q, c.total_k = total_k;
  c.s = Shape{B, H, max_Tq, max_Tk, d, block, dtype, scale};
  c.flags = flags, c.stream = stream;
  return attention(c);
}

int scfa_attn_bwd_dq_varlen(const void *q, const void *k, const void *v, const void *o, const float *lse,
                            const void *dout, const int32_t *q_offsets, const int32_t *k_offsets, int total_q,
                            int total_k, const int32_t *q_idx, const int32_t *k_idx, const int32_t *q_hash,
                            const int32_t *k_hash, const int32_t *row_count, const int32_t *row_list, void *dq,
                            float *delta, int B, int H, int max_Tq, int max_Tk, int d, int block, float scale,
                            int dtype, unsigned flags, void *stream) {
  if (q_offsets == nullptr || k_offsets == nullptr)
    return fail(SCFA_ERR_INVALID_ARGUMENT, "q_offsets and k_offsets are required");
  AttnCall c{};
  c.kind = kBwdDq;
  c.api = kApiLists;
  c.q = q, c.k = k, c.v = v, c.o = o, c.lse = lse, c.dout = dout;
  c.q_idx = q_idx, c.k_idx = k_idx, c.q_hash = q_hash, c.k_hash = k_hash;
  c.row_cnt = row_count, c.row_list = row_list, c.dq = dq, c.delta = delta;
  c.q_off = q_offsets, c.k_off = k_offsets, c.total_q = total_q, c.total_k = total_k;
  c.s = Shape{B, H, max_Tq, max_Tk, d, block, dtype, scale};
  c.flags = flags, c.stream = stream;
  return attention(c);
}

int scfa_attn_bwd_dkdv_varlen(const void *q, const void *k, const void *v, const float *lse, const void *dout,
                              const float *delta, const int32_t *q_offsets, const int32_t *k_offsets, int total_q,
                              int total_k, const int32_t *q_idx, const int32_t *k_idx, const int32_t *q_hash,
                              const int32_t *k_hash, const int32_t *col_count, const int32_t *col_list, void *dk,
                              void *dv, int B, int H, int max_Tq, int max_Tk, int d, int block, float scale,
                              int dtype, unsigned flags, void *stream) {
  if (q_offsets == nullptr || k_offsets == nullptr)
    return fail(SCFA_ERR_INVALID_ARGUMENT, "q_offsets and k_offsets are required");
  AttnCall c{};
  c.kind = kBwdDkdv;
  c.api = kApiLists;
  c.q = q, c.k = k, c.v = v, c.lse = lse, c.dout = dout, c.delta = const_cast<float *>(delta);
  c.q_idx = q_idx, c.k_idx = k_idx, c.q_hash = q_hash, c.k_hash = k_hash;
  c.col_cnt = col_count, c.col_list = col_list, c.dk = dk, c.dv = dv;
  c.q_off = q_offsets, c.k_off = k_offsets, c.total_q = total_q, c.total_k = total_k;
  c.s = Shape{B, H, max_Tq, max_Tk, d, block, dtype, scale};
  c.flags = flags, c.stream = stream;
  return attention(c);
}

int scfa_tile_slots(const int32_t *row_count, const int32_t *row_list, const int32_t *col_count,
                    const int32_t *col_list, int B, int H, int Tq, int Tk, int block, int32_t *col_base,
                    int32_t *row_slot, void *stream) {
  if (B < 1 || H < 1 || Tq < 0 || Tk < 0) return fail(SCFA_ERR_INVALID_ARGUMENT, "B, H >= 1 and Tq, Tk >= 0 required");
  if (block != 64 && block != 128) return fail(SCFA_ERR_UNSUPPORTED, "block=%d unsupported (64 or 128)", block);
  const long long BH = (long long)B * H;
  const long long nq = nblocks(Tq, block), nk = nblocks(Tk, block);
  if (BH * nq * nk >= (1ll << 31)) return fail(SCFA_ERR_INVALID_ARGUMENT, "metadata too large");
  int rc;
  if ((rc = check_ptr(row_count, BH * nq, 4, "row_count")) || (rc = check_ptr(row_list, BH * nq * nk, 4, "row_list")) ||
      (rc = check_ptr(col_count, BH * nk, 4, "col_count")) || (rc = check_ptr(col_list, BH * nk * nq, 4, "col_list")) ||
      (rc = check_ptr(col_base, BH * nk + 1, 4, "col_base")) || (rc = check_ptr(row_slot, BH * nq * nk, 4, "row_slot")))
    return rc;
  const hipError_t e = scfa::launch_tile_slots(row_count, row_list, col_count, col_list, (int)BH, (int)nq, (int)nk,
                                               col_base, row_slot, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tile slots");
  return ok();
}

int scfa_attn_bwd_prep(const void *o, const float *lse, const void *dout, const int32_t *q_rows, int Tq_src,
                       float *delta, int B, int H, int Tq, int d, int dtype, unsigned flags, void *stream) {
  if (B < 1 || H < 1 || Tq < 0 || Tq_src < 0)
    return fail(SCFA_ERR_INVALID_ARGUMENT, "B, H >= 1 and Tq, Tq_src >= 0 required");
  if (d != 64 && d != 128) return fail(SCFA_ERR_UNSUPPORTED, "head dim d=%d unsupported (64 or 128)", d);
  if (dtype != SCFA_DTYPE_BF16) return fail(SCFA_ERR_UNSUPPORTED, "scfa_attn_bwd_prep needs dtype bf16");
  if (flags & ~SCFA_FLAG_ORIG_ROWS) return fail(SCFA_ERR_INVALID_ARGUMENT, "unknown flags 0x%x", flags);
  const bool orig_rows = (flags & SCFA_FLAG_ORIG_ROWS) != 0;
  if (orig_rows && q_rows == nullptr && B * H * (long long)Tq > 0)
    return fail(SCFA_ERR_INVALID_ARGUMENT, "SCFA_FLAG_ORIG_ROWS needs q_rows");
  const int Tqs = Tq_src > 0 ? Tq_src : Tq, Tqo = orig_rows ? Tqs : Tq;
  if (q_rows == nullptr && Tqs != Tq) return fail(SCFA_ERR_INVALID_ARGUMENT, "Tq_src other than Tq needs q_rows");
  const long long BH = (long long)B * H;
  if (BH * (Tq > Tqs ? Tq : Tqs) * d >= (1ll << 31))
    return fail(SCFA_ERR_INVALID_ARGUMENT, "B*H*max(Tq,Tq_src)*d must be < 2^31");
  int rc;
  if ((rc = check_ptr(o, BH * Tqo * d, 16, "o")) || (rc = check_ptr(lse, BH * Tqo, 4, "lse")) ||
      (rc = check_ptr(dout, BH * Tqs * d, 16, "dout")) || (rc = check_ptr(q_rows, q_rows ? BH * Tq : 0, 4, "q_rows")) ||
      (rc = check_ptr(delta, 2 * BH * Tq, 4, "delta")))
    return rc;
  scfa::AttnArgs a{};
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.q_rows = q_rows;
  a.delta = delta;
  a.BH = (int)BH;
  a.Tq = Tq;
  a.Tqs = Tqs;
  a.Tqo = Tqo;
  a.d = d;
  a.delta_half = BH * Tq;
  a.orig_rows = orig_rows ? 1 : 0;
  const hipError_t e = scfa::launch_attn_bwd_prep(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "backward preprocess");
  return ok();
}

int scfa_attn_bwd_dkdv_ds_lists(const void *q, const void *k, const void *v, const float *lse, const void *dout,
                                const float *delta, const int32_t *q_idx, const int32_t *k_idx, const int32_t *q_hash,
                                const int32_t *k_hash, const int32_t *q_rows, const int32_t *k_rows, int Tq_src, int Tk_src,
                                const int32_t *col_count, const int32_t *col_list, const int32_t *col_base, void *ds,
                                long long ds_tiles, void *dk, void *dv, int B, int H, int Tq, int Tk, int d, int block,
                                float scale, int dtype, unsigned flags, void *stream) {
  AttnCall c{};
  c.kind = kBwdDkdv;
  c.api = kApiLists;
  c.q = q, c.k = k, c.v = v, c.lse = lse, c.dout = dout, c.delta = const_cast<float *>(delta);
  c.q_idx = q_idx, c.k_idx = k_idx, c.q_hash = q_hash, c.k_hash = k_hash;
  c.q_rows = q_rows, c.k_rows = k_rows, c.Tq_src = Tq_src, c.Tk_src = Tk_src;
  c.col_cnt = col_count, c.col_list = col_list, c.dk = dk, c.dv = dv;
  c.ds_path = true, c.ds = ds, c.ds_tiles = ds_tiles, c.col_base = col_base;
  c.s = Shape{B, H, Tq, Tk, d, block, dtype, scale};
  c.flags = flags, c.stream = stream;
  return attention(c);
}

int scfa_attn_bwd_dq_ds_lists(const void *q, const void *k, const void *v, const void *o, const float *lse,
                              const void *dout, const int32_t *q_idx, const int32_t *k_idx, const int32_t *q_hash,
                              const int32_t *k_hash, const int32_t *q_rows, const int32_t *k_rows, int Tq_src, int Tk_src,
                              const int32_t *row_count, const int32_t *row_list, const int32_t *row_slot,
                              const int32_t *col_base, const void *ds, long long ds_tiles, void *dq, float *delta,
                              int B, int H, int Tq, int Tk, int d, int block, float scale, int dtype, unsigned flags,
                              void *stream) {
  AttnCall c{};
  c.kind = kBwdDq;
  c.api = kApiLists;
  c.q = q, c.k = k, c.v = v, c.o = o, c.lse = lse, c.dout = dout;
  c.q_idx = q_idx, c.k_idx = k_idx, c.q_hash = q_hash, c.k_hash = k_hash;
  c.q_rows = q_rows, c.k_rows = k_rows, c.Tq_src = Tq_src, c.Tk_src = Tk_src;
  c.row_cnt = row_count, c.row_list = row_list, c.dq = dq, c.delta = delta;
  c.ds_path = true, c.ds = const_cast<void *>(ds), c.ds_tiles = ds_tiles, c.row_slot = row_slot, c.col_base = col_base;
  c.s = Shape{B, H, Tq, Tk, d, block, dtype, scale};
  c.flags = flags, c.stream = stream;
  return attention(c);
}

int scfa_lsh_bucket_sort(const void *x, const int32_t *x_rows, int T_x, const int32_t *idx, const float *R,
                         int n_buckets, int B, int H, int T, int d, int dtype, unsigned flags, int32_t *hash_sorted,
                         int32_t *idx_sorted, int32_t *perm, void *x_sorted, const void *companion,
                         void *companion_sorted, void *workspace, size_t workspace_bytes, void *stream) {
  if (B < 1 || H < 1 || T < 0 || T_x < 0) return fail(SCFA_ERR_INVALID_ARGUMENT, "B, H must be >= 1 and T, T_x >= 0");
  const int Tx = T_x > 0 ? T_x : T;
  if (x_rows == nullptr && Tx != T) return fail(SCFA_ERR_INVALID_ARGUMENT, "T_x other than T needs x_rows");
  if (x_rows && (x_sorted || companion))
    return fail(SCFA_ERR_UNSUPPORTED, "x_rows: no x_sorted / companion copies (gather the rows instead)");
  if (d != 64 && d != 128) return fail(SCFA_ERR_UNSUPPORTED, "head dim d=%d unsupported (64 or 128)", d);
  if (dtype != SCFA_DTYPE_BF16 && dtype != SCFA_DTYPE_FP32) return fail(SCFA_ERR_UNSUPPORTED, "dtype=%d unsupported", dtype);
  if (n_buckets < 2 || n_buckets > 1024 || (n_buckets & 1))
    return fail(SCFA_ERR_UNSUPPORTED, "n_buckets=%d unsupported (even, 2..1024)", n_buckets);
  if (flags & ~SCFA_FLAG_IDX_ASCENDING) return fail(SCFA_ERR_INVALID_ARGUMENT, "unknown flags 0x%x", flags);
  if ((long long)B * H * T * d >= (1ll << 31)) return fail(SCFA_ERR_INVALID_ARGUMENT, "B*H*T*d must be < 2^31");
  // rows of x are addressed in 64 bits (only the sequences' own arrays need 32-bit indices)
  if ((long long)B * H * Tx * d >= (1ll << 40)) return fail(SCFA_ERR_INVALID_ARGUMENT, "B*H*T_x*d must be < 2^40");
  const long long nX = (long long)B * H * T * d, nI = (long long)B * H * T;
  int rc;
  if ((rc = check_ptr(x, (long long)B * H * Tx * d, 16, "x")) ||
      (rc = check_ptr(x_rows, x_rows ? nI : 0, 4, "x_rows")) || (rc = check_ptr(idx, idx ? nI : 0, 4, "idx")) ||
      (rc = check_ptr(R, (long long)H * d * (n_buckets / 2), 4, "R")) ||
      (rc = check_ptr(hash_sorted, nI, 4, "hash_sorted")) || (rc = check_ptr(idx_sorted, nI, 4, "idx_sorted")) ||
      (rc = check_ptr(perm, nI, 4, "perm")))
    return rc;
  if (x_sorted && (rc = check_ptr(x_sorted, nX, 16, "x_sorted"))) return rc;
  if ((companion == nullptr) != (companion_sorted == nullptr))
    return fail(SCFA_ERR_INVALID_ARGUMENT, "companion and companion_sorted must both be NULL or both set");
  if (companion && ((rc = check_ptr(companion, nX, 16, "companion")) ||
                    (rc = check_ptr(companion_sorted, nX, 16, "companion_sorted"))))
    return rc;
  const size_t need = T > 0 ? lsh_ws(B, H, T, d, n_buckets) : 0;
  if ((rc = check_ws(workspace, workspace_bytes, need))) return rc;

  scfa::LshArgs a{};
  a.x = x;
  a.x_rows = x_rows;
  a.Tx = Tx;
  a.idx = idx;
  a.R = R;
  a.nb = n_buckets;
  a.B = B;
  a.H = H;
  a.T = T;
  a.d = d;
  a.dtype = dtype;
  a.idx_ascending = (flags & SCFA_FLAG_IDX_ASCENDING) ? 1 : 0;
  a.hash_sorted = hash_sorted;
  a.idx_sorted = idx_sorted;
  a.perm = perm;
  a.x_sorted = x_sorted;
  a.companion = companion;
  a.companion_sorted = companion_sorted;
  if (T > 0) {
    const size_t BH = (size_t)B * H;
    Carver cv{static_cast<char *>(workspace)};
    a.hash = cv.take<int32_t>(BH * T * 4);
    a.hist = cv.take<int32_t>(BH * scfa::sort_bins(n_buckets, true) * scfa::sort_chunks(T) * 4);
    a.tmp_idx[0] = cv.take<int32_t>(BH * T * 4);
    a.tmp_idx[1] = cv.take<int32_t>(BH * T * 4);
    a.tmp_src[0] = cv.take<int32_t>(BH * T * 4);
    a.tmp_src[1] = cv.take<int32_t>(BH * T * 4);
    a.R64 = cv.take<double>((size_t)H * d * scfa::lsh_r64_cols(n_buckets) * 8);
    a.Rf = cv.take<char>(scfa::lsh_frag_bytes(H, d, n_buckets));
    a.colnorm = cv.take<float>((size_t)H * (n_buckets / 2) * 4);
    a.fb_count = cv.take<int32_t>(4);
    a.scan_tmp = cv.take<int32_t>(2 * BH * scfa::sort_bins(n_buckets, true) * 4);
    a.fb_list = a.tmp_src[1];  // idle until the position passes, which run after the hash
  }
  hipError_t e = scfa::launch_lsh_bucket_sort(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "lsh bucket sort");
  return ok();
}

int scfa_block_meta(const int32_t *q_idx, const int32_t *k_idx, const int32_t *q_hash, const int32_t *k_hash, int B,
                    int H, int Tq, int Tk, int block, int32_t *q_stats, int32_t *k_stats, int32_t *row_count,
                    int32_t *row_list, int32_t *col_count, int32_t *col_list, void *stream) {
  return meta_call(q_idx, k_idx, q_hash, k_hash, B, H, Tq, Tk, block, q_stats, k_stats, false, row_count, row_list,
                   col_count, col_list, nullptr, 0, stream);
}

int scfa_block_meta_exact(const int32_t *q_idx, const int32_t *k_idx, const int32_t *q_hash, const int32_t *k_hash,
                          int B, int H, int Tq, int Tk, int block, int32_t *q_stats, int32_t *k_stats,
                          int32_t *row_count, int32_t *row_list, int32_t *col_count, int32_t *col_list,
                          void *workspace, size_t workspace_bytes, void *stream) {
  return meta_call(q_idx, k_idx, q_hash, k_hash, B, H, Tq, Tk, block, q_stats, k_stats, true, row_count, row_list,
                   col_count, col_list, workspace, workspace_bytes, stream);
}

int scfa_gather_rows(const void *src, const int32_t *index, void *dst, int B, int H, int T_src, int T_dst, int d,
                     int dtype, void *stream) {
  return rows_call(true, src, index, dst, B, H, T_src, T_dst, d, dtype, 0, stream);
}

int scfa_scatter_rows(const void *src, const int32_t *index, void *dst, int B, int H, int T_src, int T_dst, int d,
                      int dtype, unsigned flags, void *stream) {
  return rows_call(false, src, index, dst, B, H, T_src, T_dst, d, dtype, flags, stream);
}
int scfa_zero_rows(void *dst, const int32_t *index, int B, int H, int n, int T, int d, int dtype, void *stream) {
  if (B < 1 || H < 1 || n < 0 || T < 0 || d < 1)
    return fail(SCFA_ERR_INVALID_ARGUMENT, "B, H, d >= 1 and n, T >= 0 required");
  if (dtype != SCFA_DTYPE_BF16 && dtype != SCFA_DTYPE_FP32) return fail(SCFA_ERR_UNSUPPORTED, "dtype=%d unsupported", dtype);
  const int esize = dtype == SCFA_DTYPE_BF16 ? 2 : 4;
  if ((d * esize) % 16 != 0) return fail(SCFA_ERR_UNSUPPORTED, "row of %d bytes is not a multiple of 16", d * esize);
  if (d * esize > 4096) return fail(SCFA_ERR_UNSUPPORTED, "row of %d bytes exceeds 4096", d * esize);
  if ((long long)B * H > 65535) return fail(SCFA_ERR_UNSUPPORTED, "B*H = %lld exceeds 65535", (long long)B * H);
  const long long BH = (long long)B * H;
  const long long Tm = n > T ? n : T;
  if (BH * Tm >= (1ll << 31) || BH * Tm * d >= (1ll << 40)) return fail(SCFA_ERR_INVALID_ARGUMENT, "tensors too large");
  int rc;
  if ((rc = check_ptr(dst, BH * T * d, 16, "dst")) || (rc = check_ptr(index, BH * n, 4, "index"))) return rc;
  scfa::RowArgs r{nullptr, index, dst, (int)BH, n, T, d * esize / 16};
  const hipError_t e = scfa::launch_zero_rows(r, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "zero rows");
  return ok();
}

size_t scfa_workspace_size(int op, int B, int H, int Tq, int Tk, int d, int block, int n_buckets) {
  (void)d;
  if (B < 1 || H < 1 || Tq < 0) return 0;
  switch (op) {
    case SCFA_OP_QK_FWD:
    case SCFA_OP_HASH_FWD:
    case SCFA_OP_QK_BWD:
    case SCFA_OP_HASH_BWD:
      if (Tk < 0 || (block != 64 && block != 128)) return 0;
      return attn_ws(op == SCFA_OP_QK_BWD || op == SCFA_OP_HASH_BWD, B, H, Tq, Tk, block);
    case SCFA_OP_BLOCK_META_EXACT:
      if (Tk < 0 || (block != 64 && block != 128)) return 0;
      return scfa::meta_seg_bytes((size_t)B * H, nblocks(Tq, block), nblocks(Tk, block), block);
    case SCFA_OP_LSH_SORT:
      if (n_buckets < 2 || n_buckets > 1024 || (n_buckets & 1) || (d != 64 && d != 128)) return 0;
      return Tq > 0 ? lsh_ws(B, H, Tq, d, n_buckets) : 0;
    default:
      return 0;
  }
}

const char *scfa_last_error(void) { return g_err.c_str(); }

}  // extern "C"
