"""Bucket-collision coverage of a chunked within-bucket approximation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The summary page's Hash-sparse benchmark ("实验与结果 > Hash-Sparse",
Fig. 4 caption) states that SCFA covers every bucket collision while a
chunked LSH attention (sort tokens by bucket, split the sorted sequence into
fixed-size chunks, attend within the chunk and the previous one) loses part
of them.  Admissible pairs are those of the element mask (equal buckets, key
position <= query position).  SCFA visits all of them by construction (its
result is the exact masked attention); the chunked scheme visits the pairs
whose sorted key slot falls in the query's chunk or the chunk before it.
"""

from __future__ import annotations

import numpy as np


def admissible_counts(q_idx, k_idx, q_hash, k_hash) -> np.ndarray:
    """Per query, the number of admissible keys (same bucket, position <= the query's)."""
    q_idx, k_idx = np.asarray(q_idx), np.asarray(k_idx)
    q_hash, k_hash = np.asarray(q_hash), np.asarray(k_hash)
    n = np.zeros(q_idx.size, dtype=np.int64)
    for h in np.unique(q_hash):
        qs = np.nonzero(q_hash == h)[0]
        pos = np.sort(k_idx[k_hash == h])
        n[qs] = np.searchsorted(pos, q_idx[qs], side="right")
    return n


def chunked_coverage(q_idx, k_idx, q_hash, k_hash, chunk: int) -> float:
    """Fraction of admissible pairs a chunked scheme visits.

    Q and K are each ordered by (bucket, position); query slot s sees the
    keys in slots [c*(s//c - 1), c*(s//c + 1)) of the K order, c = chunk.
    """
    q_idx, k_idx = np.asarray(q_idx), np.asarray(k_idx)
    q_hash, k_hash = np.asarray(q_hash), np.asarray(k_hash)
    qo = np.lexsort((q_idx, q_hash))
    ko = np.lexsort((k_idx, k_hash))
    qi, qh = q_idx[qo], q_hash[qo]
    ki, kh = k_idx[ko], k_hash[ko]
    total = int(admissible_counts(q_idx, k_idx, q_hash, k_hash).sum())
    if total == 0:
        return 1.0
    seen = 0
    for c0 in range(0, qi.size, chunk):
        c1 = min(c0 + chunk, qi.size)
        k0, k1 = max(0, c0 - chunk), min(ki.size, c0 + chunk)
        ok = (kh[None, k0:k1] == qh[c0:c1, None]) & (ki[None, k0:k1] <= qi[c0:c1, None])
        seen += int(ok.sum())
    return seen / total
