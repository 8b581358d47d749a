"""ctypes loader for libscfa.so, the HIP library (C ABI declared in include/scfa.h).

There is no fallback: if the library is missing the import of the binding
fails loudly.  Build it with ``python -m sparse_causal_attention_amd.build``
(or ``__graft_entry__.build()``).
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libscfa.so")

# Names declared in include/scfa.h, in declaration order.
EXPORTED = (
    "scfa_qk_sparse_fwd",
    "scfa_qk_sparse_bwd",
    "scfa_hash_sparse_fwd",
    "scfa_hash_sparse_bwd",
    "scfa_hash_sparse_fwd_noalloc",
    "scfa_noalloc_scratch_bytes",
    "scfa_lsh_bucket_sort",
    "scfa_block_meta",
    "scfa_block_meta_exact",
    "scfa_attn_fwd_lists",
    "scfa_attn_bwd_dq_lists",
    "scfa_attn_bwd_dkdv_lists",
    "scfa_block_meta_varlen",
    "scfa_attn_fwd_varlen",
    "scfa_attn_bwd_dq_varlen",
    "scfa_attn_bwd_dkdv_varlen",
    "scfa_tile_slots",
    "scfa_attn_bwd_prep",
    "scfa_attn_bwd_dkdv_ds_lists",
    "scfa_attn_bwd_dq_ds_lists",
    "scfa_gather_rows",
    "scfa_scatter_rows",
    "scfa_zero_rows",
    "scfa_workspace_size",
    "scfa_last_error",
)

OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_UNSUPPORTED = 2
ERR_WORKSPACE_TOO_SMALL = 3
ERR_HIP = 4

DTYPE_BF16 = 0
DTYPE_FP32 = 1

FLAG_NO_PRUNE = 1 << 0
FLAG_FORCE_MASK = 1 << 1
FLAG_IDX_ASCENDING = 1 << 2
FLAG_ZERO_FILL = 1 << 3
FLAG_ORIG_ROWS = 1 << 4

OP_QK_FWD = 0
OP_QK_BWD = 1
OP_HASH_FWD = 2
OP_HASH_BWD = 3
OP_LSH_SORT = 4
OP_BLOCK_META_EXACT = 5

_p = ctypes.c_void_p
_i = ctypes.c_int
_u = ctypes.c_uint
_f = ctypes.c_float
_sz = ctypes.c_size_t
_i64 = ctypes.c_longlong

_ATTN_TAIL = [_i, _i, _i, _i, _i, _i, _f, _i, _u, _p, _sz, _p]
_LISTS_TAIL = [_i, _i, _i, _i, _i, _i, _f, _i, _u, _p]

_SIGNATURES = {
    "scfa_qk_sparse_fwd": [_p, _p, _p, _p, _p, _p, _p] + _ATTN_TAIL,
    "scfa_qk_sparse_bwd": [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p] + _ATTN_TAIL,
    "scfa_hash_sparse_fwd": [_p, _p, _p, _p, _p, _p, _p, _p, _p] + _ATTN_TAIL,
    "scfa_hash_sparse_bwd": [_p] * 13 + _ATTN_TAIL,
    "scfa_hash_sparse_fwd_noalloc": [_p] * 9 + _LISTS_TAIL,
    "scfa_noalloc_scratch_bytes": [],
    "scfa_lsh_bucket_sort": [_p, _p, _i, _p, _p, _i, _i, _i, _i, _i, _i, _u, _p, _p, _p, _p, _p, _p, _p, _sz, _p],
    "scfa_block_meta": [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p],
    "scfa_block_meta_exact": [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _sz, _p],
    "scfa_attn_fwd_lists": [_p] * 9 + [_i, _i] + [_p] * 4 + _LISTS_TAIL,
    "scfa_attn_bwd_dq_lists": [_p] * 12 + [_i, _i] + [_p] * 4 + _LISTS_TAIL,
    "scfa_attn_bwd_dkdv_lists": [_p] * 12 + [_i, _i] + [_p] * 4 + _LISTS_TAIL,
    "scfa_block_meta_varlen": [_p, _p, _i, _i, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _sz, _p],
    "scfa_attn_fwd_varlen": [_p, _p, _p, _p, _p, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p] + _LISTS_TAIL,
    "scfa_attn_bwd_dq_varlen": [_p] * 8 + [_i, _i] + [_p] * 8 + _LISTS_TAIL,
    "scfa_attn_bwd_dkdv_varlen": [_p] * 8 + [_i, _i] + [_p] * 8 + _LISTS_TAIL,
    "scfa_tile_slots": [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p],
    "scfa_attn_bwd_prep": [_p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _u, _p],
    "scfa_attn_bwd_dkdv_ds_lists": [_p] * 12 + [_i, _i] + [_p] * 4 + [_i64] + [_p, _p] + _LISTS_TAIL,
    "scfa_attn_bwd_dq_ds_lists": [_p] * 12 + [_i, _i] + [_p] * 5 + [_i64] + [_p, _p] + _LISTS_TAIL,
    "scfa_gather_rows": [_p, _p, _p, _i, _i, _i, _i, _i, _i, _p],
    "scfa_scatter_rows": [_p, _p, _p, _i, _i, _i, _i, _i, _i, _u, _p],
    "scfa_zero_rows": [_p, _p, _i, _i, _i, _i, _i, _i, _p],
    "scfa_workspace_size": [_i, _i, _i, _i, _i, _i, _i, _i],
    "scfa_last_error": [],
}

_LIB = None


def load() -> ctypes.CDLL:
    """Load libscfa.so once and attach the C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} not found: the HIP library is not built "
            "(run python -m sparse_causal_attention_amd.build)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    for name, argtypes in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = _i
    lib.scfa_workspace_size.restype = _sz
    lib.scfa_noalloc_scratch_bytes.restype = _sz
    lib.scfa_last_error.restype = ctypes.c_char_p
    _LIB = lib
    return lib


class ScfaError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status
        self.message = message


def check(fn: str, status: int) -> None:
    if status != OK:
        raise ScfaError(fn, status, load().scfa_last_error().decode())
