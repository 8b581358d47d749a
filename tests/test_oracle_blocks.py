"""Pins of the block-metadata oracle: closed forms, brute force, pruning soundness."""

import json
import os

import numpy as np
import pytest

from gen import WORKLOADS, keep_set
from oracle import attention as A
from oracle import blocks as Bk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tile_pairs(mask, i, j, block):
    return mask[i * block : (i + 1) * block, j * block : (j + 1) * block]


@pytest.mark.parametrize("T,block", [(64, 64), (179, 64), (1000, 64), (300, 128)])
def test_identity_positions_closed_form(T, block):
    pos = np.arange(T)
    _, _, live, free = Bk.metadata(pos, pos, None, None, block)
    n = Bk.n_blocks(T, block)
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    np.testing.assert_array_equal(live, j <= i)
    np.testing.assert_array_equal(free, j < i)


def test_shared_increasing_keep_set_closed_form():
    rng = np.random.default_rng(1)
    keep = np.sort(rng.choice(5000, 1333, replace=False))
    _, _, live, free = Bk.metadata(keep, keep, None, None, 64)
    n = Bk.n_blocks(1333, 64)
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    np.testing.assert_array_equal(live, j <= i)
    np.testing.assert_array_equal(free, j < i)


def test_workload1_golden_lists():
    g = json.load(open(os.path.join(GOLDEN, "workload1_blocks.json")))
    keep, _ = keep_set(WORKLOADS[1], 0, 0)
    assert keep.shape == (g["Tq"],)
    qs, ks, live, free = Bk.metadata(keep, keep, None, None, g["block"])
    assert [min(g["block"], g["Tq"] - b * g["block"]) for b in range(qs.shape[0])] == g["block_rows"]
    assert Bk.row_lists(live, free) == [[tuple(e) for e in r] for r in g["row_lists"]]
    assert Bk.col_lists(live, free) == [[tuple(e) for e in r] for r in g["col_lists"]]
    assert int(live.sum()) == g["live_tiles"]


def _random_case(rng, hashed, Tq, Tk, nb=4, sort_by_hash=True):
    qi = np.sort(rng.choice(3 * max(Tq, Tk), Tq, replace=False))
    ki = np.sort(rng.choice(3 * max(Tq, Tk), Tk, replace=False))
    qh = kh = None
    if hashed:
        qh, kh = rng.integers(0, nb, Tq), rng.integers(0, nb, Tk)
        if sort_by_hash:
            oq, ok = np.lexsort((qi, qh)), np.lexsort((ki, kh))
            qi, qh, ki, kh = qi[oq], qh[oq], ki[ok], kh[ok]
    return qi, ki, qh, kh


@pytest.mark.parametrize("hashed", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_liveness_is_sound_and_maskfree_is_exact(hashed, seed):
    """Every tile holding an admissible pair is live; mask-free iff all real pairs admissible."""
    rng = np.random.default_rng(seed)
    Tq, Tk, block = 333, 291, 32
    qi, ki, qh, kh = _random_case(rng, hashed, Tq, Tk, sort_by_hash=(seed != 2))
    mask = A.element_mask(qi, ki, qh, kh)
    _, _, live, free = Bk.metadata(qi, ki, qh, kh, block)
    for i in range(live.shape[0]):
        for j in range(live.shape[1]):
            t = _tile_pairs(mask, i, j, block)
            if t.any():
                assert live[i, j]
            assert free[i, j] == bool(t.all())
            if free[i, j]:
                assert live[i, j]
    if not hashed:
        # without buckets the block rule is exact: live iff some pair admissible
        for i in range(live.shape[0]):
            for j in range(live.shape[1]):
                assert live[i, j] == bool(_tile_pairs(mask, i, j, block).any())


def test_single_bucket_blocks_make_liveness_exact():
    """When every block holds one bucket, live iff the tile holds an admissible pair."""
    rng = np.random.default_rng(8)
    block = 16
    qh = np.repeat(rng.integers(0, 3, 12), block)
    kh = np.repeat(rng.integers(0, 3, 12), block)
    qi = rng.permutation(400)[: qh.size]
    ki = rng.permutation(400)[: kh.size]
    mask = A.element_mask(qi, ki, qh, kh)
    _, _, live, _ = Bk.metadata(qi, ki, qh, kh, block)
    for i in range(12):
        for j in range(12):
            assert live[i, j] == bool(_tile_pairs(mask, i, j, block).any())


@pytest.mark.parametrize("hashed", [False, True])
def test_pruned_evaluation_equals_full_mask(hashed):
    rng = np.random.default_rng(12 + hashed)
    Tq, Tk, d, block = 410, 390, 16, 64
    qi, ki, qh, kh = _random_case(rng, hashed, Tq, Tk, nb=6)
    q, k, v = (rng.standard_normal((n, d)) for n in (Tq, Tk, Tk))
    o, lse = A.forward(q, k, v, qi, ki, qh, kh)
    o2, lse2 = Bk.forward_live_tiles_only(q, k, v, qi, ki, qh, kh, block)
    np.testing.assert_allclose(o2, o, atol=1e-12, rtol=0)
    finite = np.isfinite(lse)
    np.testing.assert_array_equal(np.isfinite(lse2), finite)
    np.testing.assert_allclose(lse2[finite], lse[finite], atol=1e-12, rtol=0)


def test_block_stats_use_real_rows_only():
    idx = np.array([5, 1, 9, 3, 7, 2, 8])
    hs = np.array([2, 2, 0, 1, 3, 3, 1])
    st = Bk.block_stats(idx, hs, 3)
    np.testing.assert_array_equal(st, [[1, 9, 0, 2], [2, 7, 1, 3], [8, 8, 1, 1]])


def test_lists_are_ascending_and_consistent():
    rng = np.random.default_rng(4)
    qi, ki, qh, kh = _random_case(rng, True, 500, 500, nb=3)
    _, _, live, free = Bk.metadata(qi, ki, qh, kh, 32)
    rows, cols = Bk.row_lists(live, free), Bk.col_lists(live, free)
    pairs_r = {(i, j, f) for i, r in enumerate(rows) for j, f in r}
    pairs_c = {(i, j, f) for j, c in enumerate(cols) for i, f in c}
    assert pairs_r == pairs_c and len(pairs_r) == int(live.sum())
    for r in rows:
        assert [j for j, _ in r] == sorted(j for j, _ in r)


# ---------------------------------------------------------------------------
# Exact liveness ("2. Hash-Sparse" rules 1 and 2 read literally: a tile is kept
# iff a query and a key of it share a bucket in causal order, i.e. iff it holds
# an admissible pair).  ``tile_has_pair`` reduces the element mask per tile; the
# pins below check it by explicit per-pair loops, closed forms and a worked case.
# ---------------------------------------------------------------------------
def _tile_has_pair_loops(qi, ki, qh, kh, block):
    """Scalar loops over every (query, key) pair, written from the rule directly."""
    nq, nk = Bk.n_blocks(len(qi), block), Bk.n_blocks(len(ki), block)
    out = np.zeros((nq, nk), dtype=bool)
    for r in range(len(qi)):
        for c in range(len(ki)):
            same = qh is None or int(qh[r]) == int(kh[c])
            if same and int(ki[c]) <= int(qi[r]):
                out[r // block, c // block] = True
    return out


@pytest.mark.parametrize("seed,nb,block,sort_by_hash", [(0, 4, 16, True), (1, 6, 16, True), (2, 3, 8, False),
                                                        (3, 40, 16, True), (4, 2, 32, True), (5, 70, 16, False)])
def test_exact_liveness_equals_pair_loops(seed, nb, block, sort_by_hash):
    """Any number of buckets per block (up to every row its own bucket): the tile is
    live iff some pair in it is admissible; always a subset of the range rule."""
    rng = np.random.default_rng(100 + seed)
    Tq, Tk = 101, 87
    qi, ki, qh, kh = _random_case(rng, True, Tq, Tk, nb=nb, sort_by_hash=sort_by_hash)
    _, _, live_range, free = Bk.metadata(qi, ki, qh, kh, block)
    _, _, live, free_x = Bk.metadata_exact(qi, ki, qh, kh, block)
    np.testing.assert_array_equal(live, _tile_has_pair_loops(qi, ki, qh, kh, block))
    assert not (live & ~live_range).any()
    np.testing.assert_array_equal(free_x, free)
    assert not (free & ~live).any()


@pytest.mark.parametrize("seed", [0, 1])
def test_exact_liveness_without_buckets_is_the_range_rule(seed):
    """QK-sparse: the pair (query with the largest position, key with the smallest) is
    admissible whenever max q_idx >= min k_idx, so the block rule is already exact."""
    rng = np.random.default_rng(50 + seed)
    qi, ki, _, _ = _random_case(rng, False, 301, 277)
    if seed == 1:
        qi, ki = rng.permutation(qi), rng.permutation(ki)
    _, _, live_range, _ = Bk.metadata(qi, ki, None, None, 32)
    _, _, live, _ = Bk.metadata_exact(qi, ki, None, None, 32)
    np.testing.assert_array_equal(live, live_range)
    np.testing.assert_array_equal(live, _tile_has_pair_loops(qi, ki, None, None, 32))


def test_exact_liveness_identity_positions_one_bucket():
    """Identity positions, one bucket: live iff j <= i (standard causal tiles)."""
    pos = np.arange(200)
    h = np.zeros(200, dtype=np.int64)
    live = Bk.tile_has_pair(pos, pos, h, h, 64)
    n = Bk.n_blocks(200, 64)
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    np.testing.assert_array_equal(live, j <= i)


def test_exact_liveness_drops_bucket_matched_acausal_tiles():
    """A worked case: both blocks hold buckets {0, 1}, bucket ranges overlap and the
    blocks are causal overall, yet bucket 0 keys follow bucket 0 queries and
    bucket 1 keys follow bucket 1 queries: no valid pair, so exact liveness drops it."""
    qi = np.array([10, 11, 50, 51])
    qh = np.array([0, 0, 1, 1])
    ki = np.array([20, 21, 60, 61])
    kh = np.array([0, 0, 1, 1])
    assert not A.element_mask(qi, ki, qh, kh).any()
    _, _, live_range, _ = Bk.metadata(qi, ki, qh, kh, 4)
    _, _, live, _ = Bk.metadata_exact(qi, ki, qh, kh, 4)
    assert live_range[0, 0] and not live[0, 0]
    # one key of bucket 1 moved before the last bucket-1 query makes the tile live
    ki2 = np.array([20, 21, 51, 61])
    _, _, live2, _ = Bk.metadata_exact(qi, ki2, qh, kh, 4)
    assert live2[0, 0] and A.element_mask(qi, ki2, qh, kh).any()
    # five buckets in one block, one shared bucket (7) in causal order: live
    qi3, qh3 = np.array([1, 2, 3, 4, 90]), np.array([3, 4, 5, 6, 7])
    ki3, kh3 = np.array([80, 81, 82, 83, 89]), np.array([8, 9, 10, 11, 7])
    assert Bk.tile_has_pair(qi3, ki3, qh3, kh3, 8)[0, 0]
    assert Bk.tile_has_pair(qi3, ki3 + 1, qh3, kh3, 8)[0, 0]  # key 90 <= query 90: a token sees itself
    assert not Bk.tile_has_pair(qi3, ki3 + 2, qh3, kh3, 8)[0, 0]


@pytest.mark.parametrize("seed", [0, 1])
def test_exact_pruned_evaluation_equals_full_mask(seed):
    rng = np.random.default_rng(30 + seed)
    Tq, Tk, d, block = 410, 390, 16, 32
    qi, ki, qh, kh = _random_case(rng, True, Tq, Tk, nb=5)
    q, k, v = (rng.standard_normal((n, d)) for n in (Tq, Tk, Tk))
    o, lse = A.forward(q, k, v, qi, ki, qh, kh)
    o2, lse2 = Bk.forward_live_tiles_only(q, k, v, qi, ki, qh, kh, block, exact=True)
    np.testing.assert_allclose(o2, o, atol=1e-12, rtol=0)
    finite = np.isfinite(lse)
    np.testing.assert_array_equal(np.isfinite(lse2), finite)
    np.testing.assert_allclose(lse2[finite], lse[finite], atol=1e-12, rtol=0)
    # and it really prunes more than the range rule on bucket-sorted inputs
    assert Bk.metadata_exact(qi, ki, qh, kh, block)[2].sum() < Bk.metadata(qi, ki, qh, kh, block)[2].sum()
