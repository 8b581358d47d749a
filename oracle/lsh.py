"""LSH bucket ids and the (bucket, original position) token order.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The summary page groups similar tokens into buckets with locality-sensitive
hashing, in the style of Reformer ("why dynamic sparsity breaks it",
Hash-Sparse item; "2. Hash-Sparse"), reorders tokens by bucket, and requires
every token to keep its original position for the causal mask ("why dynamic
sparsity breaks it", closing paragraph).  The hash itself is the
random-rotation LSH of the benchmark workloads:

* projection ``p_c = sum_k x_k * R[k, c]`` for c < nb/2, accumulated in
  float64 in increasing k.  x is bf16 or fp32 and R is fp32, so every product
  is exact in float64 and only the additions round, in this fixed order;
* ``z = [p_0 .. p_{nb/2-1}, -p_0 .. -p_{nb/2-1}]`` and the bucket is the first
  index attaining ``max z``.

Token order: ascending (bucket, original position), stable and unique because
positions are distinct within a sequence.  ``perm[s]`` is the source row of
sorted slot s.
"""

from __future__ import annotations

import ctypes
import os
from typing import Tuple

import numpy as np


def project(x: np.ndarray, R: np.ndarray) -> np.ndarray:
    """float64 [T, nb/2] with sequential accumulation over the coordinate k."""
    x = np.asarray(x, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    acc = np.zeros((x.shape[0], R.shape[1]), dtype=np.float64)
    for k in range(x.shape[1]):
        acc = acc + x[:, k : k + 1] * R[k][None, :]
    return acc


def buckets_from_projection(p: np.ndarray) -> np.ndarray:
    """First argmax of [p, -p] along the last axis, int32."""
    z = np.concatenate([p, -p], axis=1)
    return np.argmax(z, axis=1).astype(np.int32)


def buckets(x: np.ndarray, R: np.ndarray) -> np.ndarray:
    """Bucket id in [0, nb) of every row of x."""
    return buckets_from_projection(project(x, R))


def bucket_sort(bucket: np.ndarray, idx: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(perm, bucket_sorted, idx_sorted) ordering rows by (bucket, idx)."""
    bucket = np.asarray(bucket)
    idx = np.asarray(idx)
    perm = np.lexsort((idx, bucket)).astype(np.int32)
    return perm, bucket[perm].astype(np.int32), idx[perm].astype(np.int32)


# ---------------------------------------------------------------------------
# The same bucket function in plain C (oracle/lsh_ref.c), for heads too large
# for the NumPy loop.  Built by oracle/build_lsh_ref.py; it is checked
# bit-for-bit against ``buckets`` above in the oracle tests.
# ---------------------------------------------------------------------------

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblsh_ref.so")
        if not os.path.exists(path):
            from .build_lsh_ref import build

            build()
        lib = ctypes.CDLL(path)
        lib.lsh_ref_buckets.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_int,
        ]
        lib.lsh_ref_buckets.restype = None
        _LIB = lib
    return _LIB


def buckets_c(x: np.ndarray, R: np.ndarray, threads: int = 0) -> np.ndarray:
    """``buckets`` computed by the C reference loop (same arithmetic, same order)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R = np.ascontiguousarray(R, dtype=np.float32)
    T, d = x.shape
    out = np.empty(T, dtype=np.int32)
    if threads <= 0:
        threads = len(os.sched_getaffinity(0))
    _lib().lsh_ref_buckets(x.ctypes.data, R.ctypes.data, T, d, R.shape[1], out.ctypes.data, threads)
    return out
