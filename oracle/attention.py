"""Dense masked attention in float64: the exact result SCFA must reproduce.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definitions, with the summary page's sections:

* Element mask, "SCFA solution > 1. QK-Sparse", rule 2, and "2. Hash-Sparse",
  rule 3: query i may attend to key j iff the key's original position does
  not exceed the query's (a token sees itself and its past), and, in
  Hash-sparse mode, iff both carry the same bucket id.
* Within the mask the result is ordinary softmax attention with scores
  ``scale * q.k``; FlashAttention-style tiling keeps this math exact
  ("the rise of FlashAttention"), and the Hash-sparse result is exact
  within-bucket attention ("2. Hash-Sparse", closing remark).
* A query with no admissible key (possible in Hash-sparse mode, because Q and
  K are hashed separately) is not defined by the page; the reading used here
  is output 0 and log-sum-exp -inf, with zero gradient contribution.
* Gradients are analytic: dV = P^T dO, dP = dO V^T, D_i = sum_j P_ij dP_ij,
  dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.

All arrays are per head: q [Tq, d], k [Tk, d], v [Tk, dv], positions and
bucket ids are integer vectors.  Rows are processed in chunks so that large
heads do not materialise a full Tq x Tk matrix.
"""

from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

_CHUNK = 2048


def element_mask(
    q_idx: np.ndarray,
    k_idx: np.ndarray,
    q_hash: Optional[np.ndarray] = None,
    k_hash: Optional[np.ndarray] = None,
) -> np.ndarray:
    """Boolean [Tq, Tk]: k_idx[j] <= q_idx[i], and q_hash[i] == k_hash[j] if hashed."""
    q_idx = np.asarray(q_idx, dtype=np.int64)
    k_idx = np.asarray(k_idx, dtype=np.int64)
    m = k_idx[None, :] <= q_idx[:, None]
    if q_hash is not None:
        m &= np.asarray(q_hash, dtype=np.int64)[:, None] == np.asarray(k_hash, dtype=np.int64)[None, :]
    return m


def _masked_probs(s: np.ndarray, mask: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Row softmax of s restricted to mask; returns (P, lse), empty rows -> (0, -inf)."""
    nonempty = mask.any(axis=1)
    sm = np.where(mask, s, -np.inf)
    m = np.where(nonempty, sm.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(mask, np.exp(np.where(mask, s, 0.0) - m[:, None]), 0.0)
    l = e.sum(axis=1)
    safe_l = np.where(nonempty, l, 1.0)
    p = e / safe_l[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(nonempty, m + np.log(safe_l), -np.inf)
    return p, lse


def forward(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    q_idx: np.ndarray,
    k_idx: np.ndarray,
    q_hash: Optional[np.ndarray] = None,
    k_hash: Optional[np.ndarray] = None,
    scale: Optional[float] = None,
) -> Tuple[np.ndarray, np.ndarray]:
    """O [Tq, dv] and lse [Tq] of masked softmax attention for one head."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[1])
    Tq = q.shape[0]
    o = np.zeros((Tq, v.shape[1]), dtype=np.float64)
    lse = np.full(Tq, -np.inf, dtype=np.float64)
    for r0 in range(0, Tq, _CHUNK):
        r1 = min(r0 + _CHUNK, Tq)
        mask = element_mask(q_idx[r0:r1], k_idx, None if q_hash is None else q_hash[r0:r1], k_hash)
        s = scale * (q[r0:r1] @ k.T)
        p, lse[r0:r1] = _masked_probs(s, mask)
        o[r0:r1] = p @ v
    return o, lse


def backward(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    do: np.ndarray,
    q_idx: np.ndarray,
    k_idx: np.ndarray,
    q_hash: Optional[np.ndarray] = None,
    k_hash: Optional[np.ndarray] = None,
    scale: Optional[float] = None,
) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Analytic dQ, dK, dV of sum(O * dO) for one head."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[1])
    Tq = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, Tq, _CHUNK):
        r1 = min(r0 + _CHUNK, Tq)
        mask = element_mask(q_idx[r0:r1], k_idx, None if q_hash is None else q_hash[r0:r1], k_hash)
        s = scale * (q[r0:r1] @ k.T)
        p, _ = _masked_probs(s, mask)
        dv += p.T @ do[r0:r1]
        dp = do[r0:r1] @ v.T
        dsum = (p * dp).sum(axis=1)
        ds = p * (dp - dsum[:, None])
        dq[r0:r1] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r0:r1])
    return dq, dk, dv


def forward_rows(
    rows: Sequence[int],
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    q_idx: np.ndarray,
    k_idx: np.ndarray,
    q_hash: Optional[np.ndarray] = None,
    k_hash: Optional[np.ndarray] = None,
    scale: Optional[float] = None,
) -> Tuple[np.ndarray, np.ndarray]:
    """O and lse of selected query rows only, each against every key of the head.

    Identical arithmetic to ``forward`` restricted to the rows; used where the
    full head is too large for a dense evaluation.
    """
    rows = np.asarray(rows, dtype=np.int64)
    return forward(
        np.asarray(q)[rows],
        k,
        v,
        np.asarray(q_idx)[rows],
        k_idx,
        None if q_hash is None else np.asarray(q_hash)[rows],
        k_hash,
        scale,
    )


def backward_rows(
    rows: Sequence[int],
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    do: np.ndarray,
    q_idx: np.ndarray,
    k_idx: np.ndarray,
    q_hash: Optional[np.ndarray] = None,
    k_hash: Optional[np.ndarray] = None,
    scale: Optional[float] = None,
) -> np.ndarray:
    """dQ of selected query rows (dQ_i depends on row i of P and dP only)."""
    rows = np.asarray(rows, dtype=np.int64)
    dq, _, _ = backward(
        np.asarray(q)[rows],
        k,
        v,
        np.asarray(do)[rows],
        np.asarray(q_idx)[rows],
        k_idx,
        None if q_hash is None else np.asarray(q_hash)[rows],
        k_hash,
        scale,
    )
    return dq


def backward_key_rows(
    key_rows: Sequence[int],
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    do: np.ndarray,
    q_idx: np.ndarray,
    k_idx: np.ndarray,
    q_hash: Optional[np.ndarray] = None,
    k_hash: Optional[np.ndarray] = None,
    scale: Optional[float] = None,
) -> Tuple[np.ndarray, np.ndarray]:
    """dK and dV of selected key rows.

    dK_j and dV_j need P_ij and dS_ij for every query i that admits key j; each
    such query's full softmax row is evaluated (all keys), so the result equals
    the corresponding rows of ``backward``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[1])
    key_rows = np.asarray(key_rows, dtype=np.int64)
    sel = element_mask(q_idx, np.asarray(k_idx)[key_rows],
                       q_hash, None if k_hash is None else np.asarray(k_hash)[key_rows])
    qrows = np.nonzero(sel.any(axis=1))[0]
    dk = np.zeros((len(key_rows), k.shape[1]))
    dv = np.zeros((len(key_rows), v.shape[1]))
    for r0 in range(0, len(qrows), _CHUNK):
        rr = qrows[r0:r0 + _CHUNK]
        mask = element_mask(q_idx[rr], k_idx, None if q_hash is None else q_hash[rr], k_hash)
        s = scale * (q[rr] @ k.T)
        p, _ = _masked_probs(s, mask)
        dp = do[rr] @ v.T
        dsum = (p * dp).sum(axis=1)
        ds = p * (dp - dsum[:, None])
        dv += p[:, key_rows].T @ do[rr]
        dk += scale * (ds[:, key_rows].T @ q[rr])
    return dk, dv


def zero_query_forward(
    q_idx: np.ndarray,
    k_idx: np.ndarray,
    v: np.ndarray,
    q_hash: Optional[np.ndarray] = None,
    k_hash: Optional[np.ndarray] = None,
) -> Tuple[np.ndarray, np.ndarray]:
    """O and lse of every query row when Q = 0, without a Tq x Tk matrix.

    With Q = 0 every admissible score is 0, so softmax is uniform over the
    admissible keys of row i: lse_i = ln N_i and O_i is the mean of their V
    rows (N_i = 0: O_i = 0, lse_i = -inf, as in ``forward``).  N_i and the V
    sums come from the keys of row i's bucket ordered by position, with
    prefix sums, so the cost is O((Tq + Tk) log Tk) and every row of a
    million-token head can be checked.
    """
    q_idx = np.asarray(q_idx, dtype=np.int64)
    k_idx = np.asarray(k_idx, dtype=np.int64)
    v = np.asarray(v, dtype=np.float64)
    if q_hash is None:
        q_hash = np.zeros_like(q_idx)
        k_hash = np.zeros_like(k_idx)
    q_hash = np.asarray(q_hash, dtype=np.int64)
    k_hash = np.asarray(k_hash, dtype=np.int64)
    o = np.zeros((q_idx.size, v.shape[1]))
    lse = np.full(q_idx.size, -np.inf)
    for h in np.unique(q_hash):
        qs = np.nonzero(q_hash == h)[0]
        ks = np.nonzero(k_hash == h)[0]
        if ks.size == 0:
            continue
        order = ks[np.argsort(k_idx[ks], kind="stable")]
        pos = k_idx[order]
        prefix = np.vstack([np.zeros((1, v.shape[1])), np.cumsum(v[order], axis=0)])
        n = np.searchsorted(pos, q_idx[qs], side="right")  # admissible keys: position <= query's
        some = n > 0
        rows = qs[some]
        o[rows] = prefix[n[some]] / n[some][:, None]
        lse[rows] = np.log(n[some])
    return o, lse
