"""Pins of the LSH oracle: exact integer cases, accumulation order, ties, sort."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from gen import bf16_round
from oracle import lsh

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_integer_inputs_give_exact_projection_and_argmax():
    """Small integers: every partial sum is exact, so p equals the integer dot product."""
    rng = np.random.default_rng(0)
    x = rng.integers(-8, 9, (200, 64)).astype(np.float32)
    R = rng.integers(-50, 51, (64, 8)).astype(np.float32)
    p = lsh.project(x, R)
    xi = x.astype(np.int64)
    Ri = R.astype(np.int64)
    exact = xi @ Ri
    np.testing.assert_array_equal(p, exact.astype(np.float64))
    b = lsh.buckets(x, R)
    for t in range(x.shape[0]):
        z = [int(v) for v in exact[t]] + [-int(v) for v in exact[t]]
        assert b[t] == z.index(max(z))


def test_two_buckets_are_the_sign_of_the_projection():
    """nb = 2: z = [p, -p], bucket 0 iff p >= 0 (exact rational check)."""
    rng = np.random.default_rng(1)
    x = bf16_round(rng.standard_normal((500, 64), dtype=np.float32))
    r = rng.standard_normal((64, 1), dtype=np.float32)
    b = lsh.buckets(x, r)
    for t in range(0, 500, 7):
        exact = sum(Fraction(float(x[t, k])) * Fraction(float(r[k, 0])) for k in range(64))
        if abs(exact) > Fraction(1, 10**6):  # far from the rounding boundary
            assert b[t] == (0 if exact >= 0 else 1)


def _golden_vectors(g):
    x = np.zeros((1, g["d"]), dtype=np.float32)
    for k, val in g.get("x_nonzero", {}).items():
        x[0, int(k)] = val
    R = np.zeros((g["d"], g["n_buckets"] // 2), dtype=np.float32)
    for k, c, val in g.get("R_nonzero", []):
        R[k, c] = val
    return x, R


def test_accumulation_order_golden():
    g = json.load(open(os.path.join(GOLDEN, "lsh_sequential_order.json")))
    x, R = _golden_vectors(g)
    assert bf16_round(x).tobytes() == x.tobytes()  # representable in bf16
    p = lsh.project(x, R)
    assert list(p[0]) == g["expected_projection"]
    assert int(lsh.buckets(x, R)[0]) == g["expected_bucket"]
    assert int(lsh.buckets_c(x, R)[0]) == g["expected_bucket"]


def test_first_maximum_ties_golden():
    g = json.load(open(os.path.join(GOLDEN, "lsh_first_max_ties.json")))
    R = np.zeros((g["d"], g["n_buckets"] // 2), dtype=np.float32)
    R[0, 0] = R[1, 1] = 1.0
    x = np.zeros((len(g["cases"]), g["d"]), dtype=np.float32)
    for t, c in enumerate(g["cases"]):
        x[t, :2] = c["x01"]
    want = [c["bucket"] for c in g["cases"]]
    assert list(lsh.buckets(x, R)) == want
    assert list(lsh.buckets_c(x, R)) == want


@pytest.mark.parametrize("d,nb,dtype", [(64, 16, "bf16"), (64, 32, "bf16"), (128, 256, "bf16"), (64, 8, "fp32")])
def test_c_reference_matches_numpy_bit_for_bit(d, nb, dtype):
    rng = np.random.default_rng(d + nb)
    x = rng.standard_normal((3000, d), dtype=np.float32)
    if dtype == "bf16":
        x = bf16_round(x)
    R = rng.standard_normal((d, nb // 2), dtype=np.float32)
    np.testing.assert_array_equal(lsh.buckets_c(x, R), lsh.buckets(x, R))


def test_bucket_sort_matches_python_sorted():
    rng = np.random.default_rng(2)
    T = 777
    bucket = rng.integers(0, 9, T).astype(np.int32)
    idx = rng.permutation(5000)[:T].astype(np.int32)
    perm, bs, is_ = lsh.bucket_sort(bucket, idx)
    ref = [t for _, _, t in sorted((int(bucket[t]), int(idx[t]), t) for t in range(T))]
    assert list(perm) == ref
    assert sorted(perm.tolist()) == list(range(T))
    np.testing.assert_array_equal(bs, bucket[perm])
    np.testing.assert_array_equal(is_, idx[perm])
    keys = list(zip(bs.tolist(), is_.tolist()))
    assert keys == sorted(keys)


def test_all_buckets_reachable_on_gaussian_data():
    rng = np.random.default_rng(3)
    x = bf16_round(rng.standard_normal((4000, 64), dtype=np.float32))
    R = rng.standard_normal((64, 8), dtype=np.float32)
    b = lsh.buckets(x, R)
    assert set(np.unique(b).tolist()) == set(range(16))
