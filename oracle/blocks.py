"""Block metadata and tile pruning, by brute force over every block pair.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Block b of a sequence of T compact rows covers rows [b*Bs, min((b+1)*Bs, T)).
Its statistics use real rows only: min/max original position and min/max
bucket id.

Tile (i, j) pairs query block i with key block j.

* Liveness.  "SCFA solution > 1. QK-Sparse", rule 1: a tile is skipped when
  every query precedes every key, i.e. max(q_idx of block i) <
  min(k_idx of block j); so it is live iff qmax_idx >= kmin_idx.
  "2. Hash-Sparse", rules 1 and 2: keep only tiles whose query-block and
  key-block buckets match and that are not acausal.  Reading used here for a
  block that spans several buckets: the tile is live iff the two blocks'
  [min, max] bucket ranges overlap (the element mask is exact, so any superset
  of the tiles holding a valid pair gives the same result; this one is the
  definition the lists are compared against).
* Mask-free.  Every real pair of the tile is valid: kmax_idx <= qmin_idx, and
  in Hash-sparse mode both blocks hold one and the same bucket id.
* Lists.  Row list of query block i: live key blocks j in ascending order
  (forward and dQ); column list of key block j: live query blocks i in
  ascending order (dK/dV).
* Exact liveness (the literal reading of "2. Hash-Sparse" rules 1 and 2: keep
  a tile only when a query and a key of it share a bucket, in causal order).
  A tile is exactly live iff it holds at least one admissible pair of the
  element mask.  ``tile_has_pair`` evaluates that from the mask itself, with
  no summary of the blocks; in QK-sparse mode it equals the range rule.
"""

from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np

from . import attention


def n_blocks(T: int, block: int) -> int:
    return (T + block - 1) // block


def block_stats(idx: np.ndarray, hsh: Optional[np.ndarray], block: int) -> np.ndarray:
    """int64 [nblocks, 4]: (min idx, max idx, min hash, max hash) over real rows.

    Hash columns are 0 when ``hsh`` is None.
    """
    idx = np.asarray(idx, dtype=np.int64)
    T = idx.shape[0]
    nb = n_blocks(T, block)
    out = np.zeros((nb, 4), dtype=np.int64)
    for b in range(nb):
        r0, r1 = b * block, min((b + 1) * block, T)
        seg = idx[r0:r1]
        out[b, 0], out[b, 1] = seg.min(), seg.max()
        if hsh is not None:
            hs = np.asarray(hsh, dtype=np.int64)[r0:r1]
            out[b, 2], out[b, 3] = hs.min(), hs.max()
    return out


def tile_live(qs: np.ndarray, ks: np.ndarray, hash_mode: bool) -> np.ndarray:
    """bool [nq, nk] liveness of every tile."""
    nq, nk = qs.shape[0], ks.shape[0]
    live = np.zeros((nq, nk), dtype=bool)
    for i in range(nq):
        for j in range(nk):
            ok = qs[i, 1] >= ks[j, 0]
            if hash_mode:
                ok = ok and qs[i, 3] >= ks[j, 2] and qs[i, 2] <= ks[j, 3]
            live[i, j] = ok
    return live


def tile_maskfree(qs: np.ndarray, ks: np.ndarray, hash_mode: bool) -> np.ndarray:
    """bool [nq, nk]: every real (query, key) pair of the tile is admissible."""
    nq, nk = qs.shape[0], ks.shape[0]
    free = np.zeros((nq, nk), dtype=bool)
    for i in range(nq):
        for j in range(nk):
            ok = ks[j, 1] <= qs[i, 0]
            if hash_mode:
                ok = ok and qs[i, 2] == qs[i, 3] == ks[j, 2] == ks[j, 3]
            free[i, j] = ok
    return free


def row_lists(live: np.ndarray, free: np.ndarray) -> List[List[Tuple[int, bool]]]:
    """Per query block: [(j, maskfree), ...] with j ascending."""
    return [[(int(j), bool(free[i, j])) for j in np.nonzero(live[i])[0]] for i in range(live.shape[0])]


def col_lists(live: np.ndarray, free: np.ndarray) -> List[List[Tuple[int, bool]]]:
    """Per key block: [(i, maskfree), ...] with i ascending."""
    return [[(int(i), bool(free[i, j])) for i in np.nonzero(live[:, j])[0]] for j in range(live.shape[1])]


def metadata(
    q_idx: np.ndarray,
    k_idx: np.ndarray,
    q_hash: Optional[np.ndarray],
    k_hash: Optional[np.ndarray],
    block: int,
):
    """Stats, live and mask-free matrices for one head."""
    hash_mode = q_hash is not None
    qs = block_stats(q_idx, q_hash, block)
    ks = block_stats(k_idx, k_hash, block)
    return qs, ks, tile_live(qs, ks, hash_mode), tile_maskfree(qs, ks, hash_mode)


def tile_has_pair(
    q_idx: np.ndarray,
    k_idx: np.ndarray,
    q_hash: Optional[np.ndarray],
    k_hash: Optional[np.ndarray],
    block: int,
) -> np.ndarray:
    """bool [nq, nk]: tile (i, j) holds at least one admissible (query, key) pair.

    Evaluated from the element mask itself, one query block at a time: the
    mask rows of block i are reduced with ``any`` over each key block's
    columns.  This is exact liveness: "2. Hash-Sparse" rule 1 keeps the tiles
    whose buckets match, rule 2 drops the acausal ones, and a tile survives
    both on some pair exactly when that pair is admissible.
    """
    Tq, Tk = len(q_idx), len(k_idx)
    nq, nk = n_blocks(Tq, block), n_blocks(Tk, block)
    out = np.zeros((nq, nk), dtype=bool)
    if Tk == 0:
        return out
    k_block = np.arange(Tk) // block
    for i in range(nq):
        r0, r1 = i * block, min((i + 1) * block, Tq)
        m = attention.element_mask(q_idx[r0:r1], k_idx, None if q_hash is None else q_hash[r0:r1], k_hash)
        hit = m.any(axis=0)
        out[i, np.unique(k_block[hit])] = True
    return out


def metadata_exact(
    q_idx: np.ndarray,
    k_idx: np.ndarray,
    q_hash: Optional[np.ndarray],
    k_hash: Optional[np.ndarray],
    block: int,
):
    """Stats, exact live and mask-free matrices for one head (live = tile_has_pair)."""
    qs, ks, _, free = metadata(q_idx, k_idx, q_hash, k_hash, block)
    return qs, ks, tile_has_pair(q_idx, k_idx, q_hash, k_hash, block), free


def forward_live_tiles_only(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    q_idx: np.ndarray,
    k_idx: np.ndarray,
    q_hash: Optional[np.ndarray],
    k_hash: Optional[np.ndarray],
    block: int,
    scale: Optional[float] = None,
    exact: bool = False,
) -> Tuple[np.ndarray, np.ndarray]:
    """Masked attention where each query block sees only the keys of its live tiles
    (range rule, or exact liveness with ``exact``).

    Equal to ``attention.forward`` exactly when pruning drops no admissible
    pair, which is what the tile rules promise.
    """
    q = np.asarray(q, dtype=np.float64)
    if exact:
        live = metadata_exact(q_idx, k_idx, q_hash, k_hash, block)[2]
    else:
        _, _, live, _ = metadata(q_idx, k_idx, q_hash, k_hash, block)
    Tq, Tk = q.shape[0], np.asarray(k).shape[0]
    o = np.zeros((Tq, np.asarray(v).shape[1]))
    lse = np.full(Tq, -np.inf)
    for i in range(live.shape[0]):
        r0, r1 = i * block, min((i + 1) * block, Tq)
        cols = [np.arange(j * block, min((j + 1) * block, Tk)) for j in np.nonzero(live[i])[0]]
        if not cols:
            continue
        c = np.concatenate(cols)
        o[r0:r1], lse[r0:r1] = attention.forward(
            q[r0:r1], np.asarray(k)[c], np.asarray(v)[c], q_idx[r0:r1], np.asarray(k_idx)[c],
            None if q_hash is None else q_hash[r0:r1], None if k_hash is None else np.asarray(k_hash)[c],
            scale)
    return o, lse
