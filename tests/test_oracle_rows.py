"""Pins of the row gather / scatter oracle: NumPy fancy indexing (a different
code path), inverse pairs, and out-of-range handling."""

import numpy as np

from oracle import rows


def _fancy_gather(src, index):
    B, H = index.shape[:2]
    return src[np.arange(B)[:, None, None], np.arange(H)[None, :, None], index]


def test_gather_equals_fancy_indexing():
    rng = np.random.default_rng(0)
    src = rng.standard_normal((2, 3, 50, 4))
    index = rng.integers(0, 50, (2, 3, 70))
    np.testing.assert_array_equal(rows.gather_rows(src, index), _fancy_gather(src, index))


def test_scatter_of_a_permutation_inverts_gather():
    rng = np.random.default_rng(1)
    src = rng.standard_normal((2, 2, 40, 3))
    perm = np.stack([np.stack([rng.permutation(40) for _ in range(2)]) for _ in range(2)])
    sorted_rows = rows.gather_rows(src, perm)  # slot s holds source row perm[s]
    np.testing.assert_array_equal(rows.scatter_rows(sorted_rows, perm, 40), src)


def test_compaction_round_trip_zero_fills_dropped_rows():
    rng = np.random.default_rng(2)
    T = 64
    src = rng.standard_normal((1, 2, T, 8))
    keep = np.stack([np.sort(rng.choice(T, 45, replace=False)) for _ in range(2)])[None]
    compact = rows.gather_rows(src, keep)
    back = rows.scatter_rows(compact, keep, T)
    mask = np.zeros((1, 2, T), bool)
    for h in range(2):
        mask[0, h, keep[0, h]] = True
    np.testing.assert_array_equal(back[mask], src[mask])
    assert np.all(back[~mask] == 0)
    base = np.full_like(src, 7.0)
    kept_base = rows.scatter_rows(compact, keep, T, zero_fill=False, base=base)
    assert np.all(kept_base[~mask] == 7.0)


def test_out_of_range_indices():
    src = np.arange(2 * 5 * 2, dtype=np.float64).reshape(1, 2, 5, 2)
    index = np.array([[[0, -1, 5, 4], [7, 2, -3, 1]]])
    g = rows.gather_rows(src, index)
    assert np.all(g[0, 0, 1] == 0) and np.all(g[0, 0, 2] == 0) and np.all(g[0, 1, 0] == 0)
    np.testing.assert_array_equal(g[0, 0, 3], src[0, 0, 4])
    s = rows.scatter_rows(src[:, :, :4], index, 5)
    np.testing.assert_array_equal(s[0, 0, 0], src[0, 0, 0])
    np.testing.assert_array_equal(s[0, 0, 4], src[0, 0, 3])
    assert np.all(s[0, 0, 1:4] == 0)


def test_zero_rows_of_the_dropped_positions_complete_an_uncompaction():
    """Scattering the kept rows over any prior contents and then clearing the dropped rows gives the
    zero-filled scatter; the cleared rows equal NumPy boolean-mask assignment."""
    rng = np.random.default_rng(3)
    B, H, T, n = 2, 3, 90, 61
    src = rng.standard_normal((B, H, n, 5))
    keep = np.stack([np.stack([np.sort(rng.choice(T, n, replace=False)) for _ in range(H)]) for _ in range(B)])
    drop = np.stack([np.stack([np.setdiff1d(np.arange(T), keep[b, h]) for h in range(H)]) for b in range(B)])
    base = rng.standard_normal((B, H, T, 5))
    stale = rows.scatter_rows(src, keep, T, zero_fill=False, base=base)
    np.testing.assert_array_equal(rows.zero_rows(stale, drop), rows.scatter_rows(src, keep, T))
    masked = np.array(base, copy=True)
    for b in range(B):
        for h in range(H):
            m = np.zeros(T, bool)
            m[drop[b, h]] = True
            masked[b, h][m] = 0.0
    np.testing.assert_array_equal(rows.zero_rows(base, drop), masked)


def test_zero_rows_skips_out_of_range_indices():
    dst = np.ones((1, 1, 4, 2))
    out = rows.zero_rows(dst, np.array([[[-1, 4, 2, 9]]]))
    assert np.all(out[0, 0, 2] == 0) and np.all(out[0, 0, [0, 1, 3]] == 1)
    assert np.all(dst == 1)  # the input is not modified
