"""Row gather and scatter: the steps either side of the attention path.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Dropping tokens leaves compact tensors whose rows keep their original
positions, and Hash-sparse attention reorders tokens by bucket (summary page,
"why dynamic sparsity breaks it" and "SCFA solution > 1. QK-Sparse").
Gathering builds those tensors; scattering puts results back at the original
rows.  Definitions, per (b, h), written as plain loops over rows:

* gather: dst[i] = src[index[i]], a zero row when index[i] is outside
  [0, T_src);
* scatter: dst[index[i]] = src[i] for index[i] in [0, T_dst), other rows
  dropped; destination rows no index names keep their previous value, or
  are zero with ``zero_fill``;
* zero rows: dst[index[i]] = 0 for index[i] in [0, T), other indices
  skipped (the rows of dropped tokens in a full-length output).
"""

from __future__ import annotations

from typing import Optional

import numpy as np


def gather_rows(src: np.ndarray, index: np.ndarray) -> np.ndarray:
    """src [B, H, T_src, d], index [B, H, T_dst] -> [B, H, T_dst, d]."""
    B, H, Ts, d = src.shape
    Td = index.shape[2]
    dst = np.zeros((B, H, Td, d), dtype=src.dtype)
    for b in range(B):
        for h in range(H):
            for i in range(Td):
                j = int(index[b, h, i])
                if 0 <= j < Ts:
                    dst[b, h, i] = src[b, h, j]
    return dst


def scatter_rows(src: np.ndarray, index: np.ndarray, T_dst: int, zero_fill: bool = True,
                 base: Optional[np.ndarray] = None) -> np.ndarray:
    """src [B, H, T_src, d], index [B, H, T_src] -> [B, H, T_dst, d] (base: prior dst contents)."""
    B, H, Ts, d = src.shape
    if zero_fill or base is None:
        dst = np.zeros((B, H, T_dst, d), dtype=src.dtype)
    else:
        dst = np.array(base, copy=True)
    for b in range(B):
        for h in range(H):
            for i in range(Ts):
                j = int(index[b, h, i])
                if 0 <= j < T_dst:
                    dst[b, h, j] = src[b, h, i]
    return dst


def zero_rows(dst: np.ndarray, index: np.ndarray) -> np.ndarray:
    """A copy of dst [B, H, T, d] with rows index[b, h, i] (index [B, H, n]) set to zero."""
    B, H, T, d = dst.shape
    out = np.array(dst, copy=True)
    for b in range(B):
        for h in range(H):
            for i in range(index.shape[2]):
                j = int(index[b, h, i])
                if 0 <= j < T:
                    out[b, h, j] = 0
    return out
