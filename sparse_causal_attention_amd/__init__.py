"""Sparse causal flash attention (SCFA) for MI355X / gfx950.

Thin PyTorch binding over the C ABI of ``libscfa.so`` (include/scfa.h).  The
functions below only marshal arguments: they check devices, shapes and dtypes,
allocate outputs and workspace with torch (device memory), and pass raw
pointers plus torch's current HIP stream to the library.  Every step of the
computation runs in the library's HIP kernels; there is no CPU or PyTorch
fallback, and importing this package fails if the library is not built.

Semantics follow the deep-paper.org summary of arXiv 2306.01160 ("Faster
Causal Attention Over Large Sequences Through Sparse Flash Attention"):
compact Q/K/V with original positions (QK-sparse) and bucket ids
(Hash-sparse), exact attention under the element mask
``k_idx <= q_idx [and q_hash == k_hash]``.
"""

from __future__ import annotations

import math
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import (  # noqa: F401
    FLAG_FORCE_MASK,
    FLAG_IDX_ASCENDING,
    FLAG_NO_PRUNE,
    FLAG_ORIG_ROWS,
    ScfaError,
)

_LIB = _lib.load()

__all__ = [
    "qk_sparse_fwd",
    "qk_sparse_bwd",
    "hash_sparse_fwd",
    "hash_sparse_bwd",
    "hash_sparse_fwd_noalloc",
    "noalloc_scratch_bytes",
    "lsh_bucket_sort",
    "block_meta",
    "attn_fwd_lists",
    "attn_bwd_dq_lists",
    "attn_bwd_dkdv_lists",
    "block_meta_varlen",
    "attn_fwd_varlen",
    "attn_bwd_dq_varlen",
    "attn_bwd_dkdv_varlen",
    "tile_slots",
    "ds_buffer",
    "attn_bwd_prep",
    "attn_bwd_dkdv_ds_lists",
    "attn_bwd_dq_ds_lists",
    "workspace_size",
    "gather_rows",
    "scatter_rows",
    "ScfaError",
    "FLAG_NO_PRUNE",
    "FLAG_FORCE_MASK",
    "FLAG_IDX_ASCENDING",
    "FLAG_ORIG_ROWS",
]


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.DTYPE_BF16
    if t.dtype == torch.float32:
        return _lib.DTYPE_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _need(t: Optional[torch.Tensor], name: str, dtype=None, shape=None) -> None:
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def workspace_size(op: int, B: int, H: int, Tq: int, Tk: int, d: int, block: int, n_buckets: int = 0) -> int:
    return int(_LIB.scfa_workspace_size(op, B, H, Tq, Tk, d, block, n_buckets))


def _workspace(op, B, H, Tq, Tk, d, block, device, n_buckets=0, workspace=None):
    n = workspace_size(op, B, H, Tq, Tk, d, block, n_buckets)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
        return workspace, workspace.numel()
    if n == 0:
        return None, 0
    return torch.empty(n, dtype=torch.uint8, device=device), n


def _attn_shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, T, d]")
    B, H, Tq, d = q.shape
    if k.shape[:2] != (B, H) or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("k and v must be [B, H, Tk, d] matching q")
    return B, H, Tq, k.shape[2], d


def _fwd(fn_name, op, q, k, v, idx_args, block, scale, flags, workspace):
    B, H, Tq, Tk, d = _attn_shapes(q, k, v)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    for t, n, T in zip(idx_args, ("q_idx", "k_idx", "q_hash", "k_hash"), (Tq, Tk, Tq, Tk)):
        _need(t, n, torch.int32, (B, H, T))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    ws, nws = _workspace(op, B, H, Tq, Tk, d, block, q.device, workspace=workspace)
    fn = getattr(_LIB, fn_name)
    rc = fn(_ptr(q), _ptr(k), _ptr(v), *[_ptr(t) for t in idx_args], _ptr(o), _ptr(lse),
            B, H, Tq, Tk, d, block, float(scale), _dtype_code(q), int(flags), _ptr(ws), nws, _stream())
    _lib.check(fn_name, rc)
    return o, lse


def _bwd(fn_name, op, q, k, v, o, lse, dout, idx_args, block, scale, flags, workspace):
    B, H, Tq, Tk, d = _attn_shapes(q, k, v)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _need(t, n, q.dtype)
    _need(o, "o", shape=q.shape)
    _need(dout, "dout", shape=q.shape)
    _need(lse, "lse", torch.float32, (B, H, Tq))
    for t, n, T in zip(idx_args, ("q_idx", "k_idx", "q_hash", "k_hash"), (Tq, Tk, Tq, Tk)):
        _need(t, n, torch.int32, (B, H, T))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws, nws = _workspace(op, B, H, Tq, Tk, d, block, q.device, workspace=workspace)
    fn = getattr(_LIB, fn_name)
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), *[_ptr(t) for t in idx_args],
            _ptr(dq), _ptr(dk), _ptr(dv), B, H, Tq, Tk, d, block, float(scale), _dtype_code(q), int(flags),
            _ptr(ws), nws, _stream())
    _lib.check(fn_name, rc)
    return dq, dk, dv


def qk_sparse_fwd(q, k, v, q_idx=None, k_idx=None, *, block=64, scale=None, flags=0, workspace=None
                  ) -> Tuple[torch.Tensor, torch.Tensor]:
    """QK-sparse forward; q_idx = k_idx = None gives dense causal attention."""
    return _fwd("scfa_qk_sparse_fwd", _lib.OP_QK_FWD, q, k, v, (q_idx, k_idx), block, scale, flags, workspace)


def qk_sparse_bwd(q, k, v, o, lse, dout, q_idx=None, k_idx=None, *, block=64, scale=None, flags=0, workspace=None):
    """Gradients (dq, dk, dv) of sum(o * dout) for the QK-sparse forward."""
    return _bwd("scfa_qk_sparse_bwd", _lib.OP_QK_BWD, q, k, v, o, lse, dout, (q_idx, k_idx), block, scale,
                flags, workspace)


def hash_sparse_fwd(q, k, v, q_idx, k_idx, q_hash, k_hash, *, block=64, scale=None, flags=0, workspace=None):
    """Hash-sparse forward: causal on positions and restricted to equal bucket ids."""
    return _fwd("scfa_hash_sparse_fwd", _lib.OP_HASH_FWD, q, k, v, (q_idx, k_idx, q_hash, k_hash), block, scale,
                flags, workspace)


def hash_sparse_bwd(q, k, v, o, lse, dout, q_idx, k_idx, q_hash, k_hash, *, block=64, scale=None, flags=0,
                    workspace=None):
    """Gradients (dq, dk, dv) for the Hash-sparse forward."""
    return _bwd("scfa_hash_sparse_bwd", _lib.OP_HASH_BWD, q, k, v, o, lse, dout, (q_idx, k_idx, q_hash, k_hash),
                block, scale, flags, workspace)


def hash_sparse_fwd_noalloc(q, k, v, q_idx, k_idx, q_hash, k_hash, *, block=64, scale=None, flags=0, out=None):
    """hash_sparse_fwd without a workspace: the library uses its static per-GPU scratch
    (scfa_hash_sparse_fwd_noalloc).  ``out`` optionally supplies preallocated (o, lse)."""
    B, H, Tq, Tk, d = _attn_shapes(q, k, v)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    for t, n, T in zip((q_idx, k_idx, q_hash, k_hash), ("q_idx", "k_idx", "q_hash", "k_hash"), (Tq, Tk, Tq, Tk)):
        _need(t, n, torch.int32, (B, H, T))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = out if out is not None else (torch.empty_like(q),
                                          torch.empty((B, H, Tq), dtype=torch.float32, device=q.device))
    rc = _LIB.scfa_hash_sparse_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(k_idx), _ptr(q_hash),
                                           _ptr(k_hash), _ptr(o), _ptr(lse), B, H, Tq, Tk, d, block, float(scale),
                                           _dtype_code(q), int(flags), _stream())
    _lib.check("scfa_hash_sparse_fwd_noalloc", rc)
    return o, lse


def noalloc_scratch_bytes() -> int:
    """Bytes of the static per-GPU scratch of hash_sparse_fwd_noalloc."""
    return int(_LIB.scfa_noalloc_scratch_bytes())


def lsh_bucket_sort(x, R, n_buckets, idx=None, companion=None, *, idx_ascending=False, want_x=True,
                    workspace=None, x_rows=None):
    """Bucket ids of x's rows and their (bucket, idx) order.

    Returns (hash_sorted, idx_sorted, perm, x_sorted, companion_sorted); the last
    two are None when not requested.  ``x_rows`` (int32 [B,H,T]) makes token t of
    each sequence row x_rows[t] of x, whose length may differ (e.g. the kept tokens
    of full-length tensors); x_sorted and companion are then unavailable.
    """
    if x.dim() != 4:
        raise ValueError("x must be [B, H, T, d]")
    B, H, Tx, d = x.shape
    T = x_rows.shape[2] if x_rows is not None else Tx
    _need(x, "x")
    _need(x_rows, "x_rows", torch.int32, (B, H, T))
    _need(R, "R", torch.float32, (H, d, n_buckets // 2))
    _need(idx, "idx", torch.int32, (B, H, T))
    _need(companion, "companion", x.dtype, x.shape)
    if x_rows is not None and (want_x or companion is not None):
        raise ValueError("x_rows: pass want_x=False and no companion (gather the rows instead)")
    hs = torch.empty((B, H, T), dtype=torch.int32, device=x.device)
    ids = torch.empty_like(hs)
    perm = torch.empty_like(hs)
    xs = torch.empty_like(x) if want_x else None
    cs = torch.empty_like(companion) if companion is not None else None
    ws, nws = _workspace(_lib.OP_LSH_SORT, B, H, T, 0, d, 0, x.device, n_buckets=n_buckets, workspace=workspace)
    flags = _lib.FLAG_IDX_ASCENDING if idx_ascending else 0
    rc = _LIB.scfa_lsh_bucket_sort(_ptr(x), _ptr(x_rows), Tx, _ptr(idx), _ptr(R), n_buckets, B, H, T, d,
                                   _dtype_code(x), flags, _ptr(hs), _ptr(ids), _ptr(perm), _ptr(xs),
                                   _ptr(companion), _ptr(cs), _ptr(ws), nws, _stream())
    _lib.check("scfa_lsh_bucket_sort", rc)
    return hs, ids, perm, xs, cs


def block_meta(q_idx, k_idx, q_hash=None, k_hash=None, *, block=64, with_cols=True, exact=False, workspace=None):
    """Block statistics and live-tile lists (see include/scfa.h, scfa_block_meta).

    ``exact=True`` calls scfa_block_meta_exact: in Hash-sparse mode the lists
    also drop tiles that pass the bucket-range test yet hold no valid pair.
    ``workspace`` optionally supplies its scratch (uint8, see workspace_size).
    """
    B, H, Tq = q_idx.shape
    Tk = k_idx.shape[2]
    _need(q_idx, "q_idx", torch.int32)
    _need(k_idx, "k_idx", torch.int32, (B, H, Tk))
    _need(q_hash, "q_hash", torch.int32, (B, H, Tq))
    _need(k_hash, "k_hash", torch.int32, (B, H, Tk))
    nq, nk = -(-Tq // block), -(-Tk // block)
    dev = q_idx.device
    out = {
        "q_stats": torch.empty((B, H, nq, 4), dtype=torch.int32, device=dev),
        "k_stats": torch.empty((B, H, nk, 4), dtype=torch.int32, device=dev),
        "row_count": torch.empty((B, H, nq), dtype=torch.int32, device=dev),
        "row_list": torch.empty((B, H, nq, nk), dtype=torch.int32, device=dev),
    }
    if with_cols:
        out["col_count"] = torch.empty((B, H, nk), dtype=torch.int32, device=dev)
        out["col_list"] = torch.empty((B, H, nk, nq), dtype=torch.int32, device=dev)
    out["block"] = block
    lists = (_ptr(out["row_count"]), _ptr(out["row_list"]), _ptr(out.get("col_count")), _ptr(out.get("col_list")))
    if exact:
        ws, nws = (None, 0)
        if q_hash is not None:
            ws, nws = _workspace(_lib.OP_BLOCK_META_EXACT, B, H, Tq, Tk, 0, block, dev, workspace=workspace)
        rc = _LIB.scfa_block_meta_exact(_ptr(q_idx), _ptr(k_idx), _ptr(q_hash), _ptr(k_hash), B, H, Tq, Tk, block,
                                        _ptr(out["q_stats"]), _ptr(out["k_stats"]), *lists, _ptr(ws), nws,
                                        _stream())
        _lib.check("scfa_block_meta_exact", rc)
    else:
        rc = _LIB.scfa_block_meta(_ptr(q_idx), _ptr(k_idx), _ptr(q_hash), _ptr(k_hash), B, H, Tq, Tk, block,
                                  _ptr(out["q_stats"]), _ptr(out["k_stats"]), *lists, _stream())
        _lib.check("scfa_block_meta", rc)
    return out


def _list_args(meta, key_cnt, key_list):
    if meta is None:
        return None, None
    return meta[key_cnt], meta[key_list]


def _view_shapes(q, k, v, q_rows, k_rows):
    """(B, H, Tq, Tk, d, Tq_src, Tk_src): the attention's view has Tq queries and Tk keys (the lengths
    of q_rows / k_rows when given, else of q / k); q (dout) and k, v hold Tq_src and Tk_src rows per head."""
    B, H, Tqs, Tks, d = _attn_shapes(q, k, v)
    _need(q, "q")
    _need(k, "k", q.dtype)
    _need(v, "v", q.dtype)
    Tq = q_rows.shape[2] if q_rows is not None else Tqs
    Tk = k_rows.shape[2] if k_rows is not None else Tks
    _need(q_rows, "q_rows", torch.int32, (B, H, Tq))
    _need(k_rows, "k_rows", torch.int32, (B, H, Tk))
    return B, H, Tq, Tk, d, Tqs, Tks


def _rows_args(q_rows, k_rows, Tqs, Tks):
    return _ptr(q_rows), _ptr(k_rows), Tqs, Tks


def _out_rows(flags, T_view, T_src):
    """Rows per head of an output: the caller's tensor length with FLAG_ORIG_ROWS, else the view's."""
    return T_src if int(flags) & _lib.FLAG_ORIG_ROWS else T_view


def _kv_grads(k, flags, Tk, Tks):
    B, H, _, d = k.shape
    shape = (B, H, _out_rows(flags, Tk, Tks), d)
    return torch.empty(shape, dtype=k.dtype, device=k.device), torch.empty(shape, dtype=k.dtype, device=k.device)


def attn_fwd_lists(q, k, v, q_idx, k_idx, q_hash, k_hash, meta, *, block=64, scale=None, flags=0, out=None,
                   q_rows=None, k_rows=None):
    """Forward over lists from ``block_meta`` (one kernel).  Positions None = dense causal.

    ``out`` optionally supplies preallocated (o, lse).  ``q_rows`` / ``k_rows`` (int32 [B,H,Tq] /
    [B,H,Tk]) make row i of the attention's Q row q_rows[i] of q and row j of K, V row k_rows[j] of
    k, v: a reordered view without copies, or, with q and k longer than the view, the kept rows of
    full-length tensors read in place.  Outputs are indexed by the view's rows, or with
    FLAG_ORIG_ROWS by q's rows (rows no q_rows entry names are left unwritten).
    """
    B, H, Tq, Tk, d, Tqs, Tks = _view_shapes(q, k, v, q_rows, k_rows)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    To = _out_rows(flags, Tq, Tqs)
    o, lse = out if out is not None else (torch.empty((B, H, To, d), dtype=q.dtype, device=q.device),
                                          torch.empty((B, H, To), dtype=torch.float32, device=q.device))
    rc_, rl_ = _list_args(meta, "row_count", "row_list")
    rc = _LIB.scfa_attn_fwd_lists(_ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(k_idx), _ptr(q_hash), _ptr(k_hash),
                                  *_rows_args(q_rows, k_rows, Tqs, Tks), _ptr(rc_), _ptr(rl_), _ptr(o), _ptr(lse),
                                  B, H, Tq, Tk, d, block, float(scale), _dtype_code(q), int(flags), _stream())
    _lib.check("scfa_attn_fwd_lists", rc)
    return o, lse


def attn_bwd_dq_lists(q, k, v, o, lse, dout, q_idx, k_idx, q_hash, k_hash, meta, *, block=64, scale=None, flags=0,
                      out=None, q_rows=None, k_rows=None):
    """dQ over row lists (one kernel).  Returns (dq, delta) with delta [2,B,H,Tq] float32 scratch
    (rowsum(dout * o), lse * log2 e) for attn_bwd_dkdv_lists."""
    B, H, Tq, Tk, d, Tqs, Tks = _view_shapes(q, k, v, q_rows, k_rows)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, delta = out if out is not None else (
        torch.empty((B, H, _out_rows(flags, Tq, Tqs), d), dtype=q.dtype, device=q.device),
        torch.empty((2, B, H, Tq), dtype=torch.float32, device=q.device))
    rc_, rl_ = _list_args(meta, "row_count", "row_list")
    rc = _LIB.scfa_attn_bwd_dq_lists(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(q_idx),
                                     _ptr(k_idx), _ptr(q_hash), _ptr(k_hash), *_rows_args(q_rows, k_rows, Tqs, Tks),
                                     _ptr(rc_), _ptr(rl_), _ptr(dq), _ptr(delta), B, H, Tq, Tk, d, block, float(scale),
                                     _dtype_code(q), int(flags), _stream())
    _lib.check("scfa_attn_bwd_dq_lists", rc)
    return dq, delta


def attn_bwd_dkdv_lists(q, k, v, lse, dout, delta, q_idx, k_idx, q_hash, k_hash, meta, *, block=64, scale=None,
                        flags=0, out=None, q_rows=None, k_rows=None):
    """dK and dV over column lists (one kernel), reading delta from attn_bwd_dq_lists."""
    B, H, Tq, Tk, d, Tqs, Tks = _view_shapes(q, k, v, q_rows, k_rows)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dk, dv = out if out is not None else _kv_grads(k, flags, Tk, Tks)
    cc_, cl_ = _list_args(meta, "col_count", "col_list")
    rc = _LIB.scfa_attn_bwd_dkdv_lists(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(delta), _ptr(q_idx),
                                       _ptr(k_idx), _ptr(q_hash), _ptr(k_hash), *_rows_args(q_rows, k_rows, Tqs, Tks),
                                       _ptr(cc_), _ptr(cl_), _ptr(dk), _ptr(dv), B, H, Tq, Tk, d, block,
                                       float(scale), _dtype_code(q), int(flags), _stream())
    _lib.check("scfa_attn_bwd_dkdv_lists", rc)
    return dk, dv


def _varlen_check(q_off, k_off, H):
    _need(q_off, "q_offsets", torch.int32)
    _need(k_off, "k_offsets", torch.int32, q_off.shape)
    if q_off.dim() != 1 or (q_off.numel() - 1) % H:
        raise ValueError("offsets must be [B*H + 1]")
    return (q_off.numel() - 1) // H


def block_meta_varlen(q_off, k_off, q_idx, k_idx, q_hash=None, k_hash=None, *, H, max_Tq, max_Tk, block=64,
                      with_cols=True):
    """Exact block lists for packed ragged heads (scfa_block_meta_varlen).

    q_off, k_off: int32 [B*H + 1] offsets of each head's rows in the packed q_idx [total_q] / k_idx
    [total_k] (and buckets); lists are sized by max_Tq, max_Tk.
    """
    B = _varlen_check(q_off, k_off, H)
    tq, tk = q_idx.numel(), k_idx.numel()
    _need(q_idx, "q_idx", torch.int32, (tq,))
    _need(k_idx, "k_idx", torch.int32, (tk,))
    _need(q_hash, "q_hash", torch.int32, (tq,))
    _need(k_hash, "k_hash", torch.int32, (tk,))
    nq, nk = -(-max_Tq // block), -(-max_Tk // block)
    dev = q_idx.device
    out = {
        "q_stats": torch.empty((B, H, nq, 4), dtype=torch.int32, device=dev),
        "k_stats": torch.empty((B, H, nk, 4), dtype=torch.int32, device=dev),
        "row_count": torch.empty((B, H, nq), dtype=torch.int32, device=dev),
        "row_list": torch.empty((B, H, nq, nk), dtype=torch.int32, device=dev),
        "block": block,
    }
    if with_cols:
        out["col_count"] = torch.empty((B, H, nk), dtype=torch.int32, device=dev)
        out["col_list"] = torch.empty((B, H, nk, nq), dtype=torch.int32, device=dev)
    ws, nws = (None, 0)
    if q_hash is not None:
        ws, nws = _workspace(_lib.OP_BLOCK_META_EXACT, B, H, max_Tq, max_Tk, 0, block, dev)
    rc = _LIB.scfa_block_meta_varlen(_ptr(q_off), _ptr(k_off), tq, tk, _ptr(q_idx), _ptr(k_idx), _ptr(q_hash),
                                     _ptr(k_hash), B, H, max_Tq, max_Tk, block, _ptr(out["q_stats"]),
                                     _ptr(out["k_stats"]), _ptr(out["row_count"]), _ptr(out["row_list"]),
                                     _ptr(out.get("col_count")), _ptr(out.get("col_list")), _ptr(ws), nws, _stream())
    _lib.check("scfa_block_meta_varlen", rc)
    return out


def _varlen_shapes(q, k, v, q_off, k_off, H):
    B = _varlen_check(q_off, k_off, H)
    if q.dim() != 2 or k.dim() != 2 or v.shape != k.shape or k.shape[1] != q.shape[1]:
        raise ValueError("packed q [total_q, d], k and v [total_k, d]")
    return B, q.shape[0], k.shape[0], q.shape[1]


def attn_fwd_varlen(q, k, v, q_off, k_off, q_idx, k_idx, q_hash, k_hash, meta, *, H, max_Tq, max_Tk, block=64,
                    scale=None, flags=0):
    """Forward over packed ragged heads (scfa_attn_fwd_varlen); positions None = dense causal per head."""
    B, tq, tk, d = _varlen_shapes(q, k, v, q_off, k_off, H)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((tq,), dtype=torch.float32, device=q.device)
    rc_, rl_ = _list_args(meta, "row_count", "row_list")
    rc = _LIB.scfa_attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(q_off), _ptr(k_off), tq, tk, _ptr(q_idx),
                                   _ptr(k_idx), _ptr(q_hash), _ptr(k_hash), _ptr(rc_), _ptr(rl_), _ptr(o), _ptr(lse),
                                   B, H, max_Tq, max_Tk, d, block, float(scale), _dtype_code(q), int(flags), _stream())
    _lib.check("scfa_attn_fwd_varlen", rc)
    return o, lse


def attn_bwd_dq_varlen(q, k, v, o, lse, dout, q_off, k_off, q_idx, k_idx, q_hash, k_hash, meta, *, H, max_Tq,
                       max_Tk, block=64, scale=None, flags=0):
    """dQ (and delta [2, total_q]) over packed ragged heads (scfa_attn_bwd_dq_varlen)."""
    B, tq, tk, d = _varlen_shapes(q, k, v, q_off, k_off, H)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q)
    delta = torch.empty((2, tq), dtype=torch.float32, device=q.device)
    rc_, rl_ = _list_args(meta, "row_count", "row_list")
    rc = _LIB.scfa_attn_bwd_dq_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(q_off),
                                      _ptr(k_off), tq, tk, _ptr(q_idx), _ptr(k_idx), _ptr(q_hash), _ptr(k_hash),
                                      _ptr(rc_), _ptr(rl_), _ptr(dq), _ptr(delta), B, H, max_Tq, max_Tk, d, block,
                                      float(scale), _dtype_code(q), int(flags), _stream())
    _lib.check("scfa_attn_bwd_dq_varlen", rc)
    return dq, delta


def attn_bwd_dkdv_varlen(q, k, v, lse, dout, delta, q_off, k_off, q_idx, k_idx, q_hash, k_hash, meta, *, H,
                         max_Tq, max_Tk, block=64, scale=None, flags=0):
    """dK, dV over packed ragged heads (scfa_attn_bwd_dkdv_varlen), reading delta from attn_bwd_dq_varlen."""
    B, tq, tk, d = _varlen_shapes(q, k, v, q_off, k_off, H)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    cc_, cl_ = _list_args(meta, "col_count", "col_list")
    rc = _LIB.scfa_attn_bwd_dkdv_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(delta), _ptr(q_off),
                                        _ptr(k_off), tq, tk, _ptr(q_idx), _ptr(k_idx), _ptr(q_hash), _ptr(k_hash),
                                        _ptr(cc_), _ptr(cl_), _ptr(dk), _ptr(dv), B, H, max_Tq, max_Tk, d, block,
                                        float(scale), _dtype_code(q), int(flags), _stream())
    _lib.check("scfa_attn_bwd_dkdv_varlen", rc)
    return dk, dv


def tile_slots(meta):
    """Slot numbering of the live tiles for the stored-dS backward (scfa_tile_slots).

    Adds "col_base" (int32 [B*H*nk + 1], the live-tile count last) and "row_slot"
    (int32 [B,H,nq,nk]) to ``meta`` (which needs column lists) and returns it.
    """
    B, H, nq, nk = meta["row_list"].shape
    Tq_blocks, Tk_blocks = nq, nk
    dev = meta["row_list"].device
    meta["col_base"] = torch.empty(B * H * nk + 1, dtype=torch.int32, device=dev)
    meta["row_slot"] = torch.empty((B, H, nq, nk), dtype=torch.int32, device=dev)
    block = meta.get("block", 64)
    # Tq / Tk only size the lists; any lengths with these block counts give the same result
    rc = _LIB.scfa_tile_slots(_ptr(meta["row_count"]), _ptr(meta["row_list"]), _ptr(meta["col_count"]),
                              _ptr(meta["col_list"]), B, H, Tq_blocks * block, Tk_blocks * block, block,
                              _ptr(meta["col_base"]), _ptr(meta["row_slot"]), _stream())
    _lib.check("scfa_tile_slots", rc)
    return meta


def ds_buffer(n_tiles, block=64, device="cuda"):
    """A dS buffer of n_tiles tiles (bf16 [n_tiles, block, block]) for the stored-dS backward."""
    return torch.empty((max(int(n_tiles), 0), block, block), dtype=torch.bfloat16, device=device)


def attn_bwd_prep(o, lse, dout, *, q_rows=None, out=None, flags=0):
    """delta [2,B,H,Tq] float32 = (rowsum(dout * o), lse * log2 e) (scfa_attn_bwd_prep); flags may hold
    FLAG_ORIG_ROWS (o and lse at the caller's rows).  dout [B,H,Tq_src,d] is read through q_rows."""
    if dout.dim() != 4:
        raise ValueError("dout must be [B, H, T, d]")
    B, H, Tqs, d = dout.shape
    Tq = q_rows.shape[2] if q_rows is not None else Tqs
    To = _out_rows(flags, Tq, Tqs)
    _need(dout, "dout", torch.bfloat16)
    _need(o, "o", torch.bfloat16, (B, H, To, d))
    _need(lse, "lse", torch.float32, (B, H, To))
    _need(q_rows, "q_rows", torch.int32, (B, H, Tq))
    delta = out if out is not None else torch.empty((2, B, H, Tq), dtype=torch.float32, device=o.device)
    rc = _LIB.scfa_attn_bwd_prep(_ptr(o), _ptr(lse), _ptr(dout), _ptr(q_rows), Tqs, _ptr(delta), B, H, Tq, d,
                                 _dtype_code(o), int(flags), _stream())
    _lib.check("scfa_attn_bwd_prep", rc)
    return delta


def attn_bwd_dkdv_ds_lists(q, k, v, lse, dout, delta, q_idx, k_idx, q_hash, k_hash, meta, ds, *, block=64,
                           scale=None, flags=0, out=None, q_rows=None, k_rows=None):
    """dK, dV over column lists, storing every live tile's dS in ``ds`` (needs tile_slots(meta))."""
    B, H, Tq, Tk, d, Tqs, Tks = _view_shapes(q, k, v, q_rows, k_rows)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _need(ds, "ds", torch.bfloat16)
    dk, dv = out if out is not None else _kv_grads(k, flags, Tk, Tks)
    rc = _LIB.scfa_attn_bwd_dkdv_ds_lists(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(delta),
                                          _ptr(q_idx), _ptr(k_idx), _ptr(q_hash), _ptr(k_hash),
                                          *_rows_args(q_rows, k_rows, Tqs, Tks), _ptr(meta["col_count"]),
                                          _ptr(meta["col_list"]), _ptr(meta["col_base"]), _ptr(ds),
                                          ds.shape[0] if ds.dim() == 3 else 0, _ptr(dk), _ptr(dv), B, H, Tq, Tk, d,
                                          block, float(scale), _dtype_code(q), int(flags), _stream())
    _lib.check("scfa_attn_bwd_dkdv_ds_lists", rc)
    return dk, dv


def attn_bwd_dq_ds_lists(q, k, v, o, lse, dout, q_idx, k_idx, q_hash, k_hash, meta, ds, delta, *, block=64,
                         scale=None, flags=0, out=None, q_rows=None, k_rows=None):
    """dQ from the stored dS tiles (after attn_bwd_dkdv_ds_lists); falls back to recomputing when the
    buffer was too small for every live tile."""
    B, H, Tq, Tk, d, Tqs, Tks = _view_shapes(q, k, v, q_rows, k_rows)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _need(ds, "ds", torch.bfloat16)
    dq = out if out is not None else torch.empty((B, H, _out_rows(flags, Tq, Tqs), d), dtype=q.dtype,
                                                 device=q.device)
    rc = _LIB.scfa_attn_bwd_dq_ds_lists(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(q_idx),
                                        _ptr(k_idx), _ptr(q_hash), _ptr(k_hash), *_rows_args(q_rows, k_rows, Tqs, Tks),
                                        _ptr(meta["row_count"]), _ptr(meta["row_list"]), _ptr(meta["row_slot"]),
                                        _ptr(meta["col_base"]), _ptr(ds), ds.shape[0] if ds.dim() == 3 else 0,
                                        _ptr(dq), _ptr(delta), B, H, Tq, Tk, d, block, float(scale),
                                        _dtype_code(q), int(flags), _stream())
    _lib.check("scfa_attn_bwd_dq_ds_lists", rc)
    return dq


def gather_rows(src, index, *, out=None):
    """dst[b, h, i] = src[b, h, index[b, h, i]] (zero rows for out-of-range indices).

    Compaction of kept tokens (index = their positions) or reordering (index =
    a sort permutation).  src [B,H,T_src,d]; index [B,H,T_dst] int32.  ``out``
    optionally supplies dst (contiguous [B,H,T_dst,d], e.g. a slice of a larger
    allocation along B).
    """
    B, H, Ts, d = src.shape
    _need(src, "src")
    Td = index.shape[2]
    _need(index, "index", torch.int32, (B, H, Td))
    _need(out, "out", src.dtype, (B, H, Td, d))
    dst = out if out is not None else torch.empty((B, H, Td, d), dtype=src.dtype, device=src.device)
    rc = _LIB.scfa_gather_rows(_ptr(src), _ptr(index), _ptr(dst), B, H, Ts, Td, d, _dtype_code(src), _stream())
    _lib.check("scfa_gather_rows", rc)
    return dst


def zero_rows(dst, index):
    """dst[b, h, index[b, h, i]] = 0 in place (out-of-range indices skipped); returns dst.

    Clears the dropped positions of full-length outputs whose kept rows the attention wrote in place
    (FLAG_ORIG_ROWS with full-length q, k, v).  dst [B,H,T,d]; index [B,H,n] int32.
    """
    B, H, T, d = dst.shape
    _need(dst, "dst")
    n = index.shape[2]
    _need(index, "index", torch.int32, (B, H, n))
    rc = _LIB.scfa_zero_rows(_ptr(dst), _ptr(index), B, H, n, T, d, _dtype_code(dst), _stream())
    _lib.check("scfa_zero_rows", rc)
    return dst


def scatter_rows(src, index, T_dst, *, zero_fill=True, out=None):
    """dst[b, h, index[b, h, i]] = src[b, h, i]; rows no index names are 0 with ``zero_fill``.

    Un-sorting (index = the sort permutation, T_dst = T_src) or un-compaction
    (index = kept positions, T_dst = original length).  src [B,H,T_src,d].
    """
    B, H, Ts, d = src.shape
    _need(src, "src")
    _need(index, "index", torch.int32, (B, H, Ts))
    dst = out if out is not None else torch.empty((B, H, T_dst, d), dtype=src.dtype, device=src.device)
    flags = _lib.FLAG_ZERO_FILL if zero_fill else 0
    rc = _LIB.scfa_scatter_rows(_ptr(src), _ptr(index), _ptr(dst), B, H, Ts, T_dst, d, _dtype_code(src), flags,
                                _stream())
    _lib.check("scfa_scatter_rows", rc)
    return dst
