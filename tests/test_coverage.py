"""Bucket-collision coverage: SCFA's exact mask versus a chunked within-bucket
approximation (CPU measurement; the GPU side of SCFA's 100 % is the Q = 0
closed-form check on every row in test_gpu_workloads.py)."""

import numpy as np
import pytest

from gen import WORKLOADS, head_inputs, lsh_rotation
from oracle import attention as A
from oracle import coverage as C
from oracle import lsh


def test_admissible_counts_and_chunked_coverage_brute_force():
    rng = np.random.default_rng(4)
    T = 300
    qi = ki = np.arange(T)
    qh, kh = rng.integers(0, 6, T), rng.integers(0, 6, T)
    mask = A.element_mask(qi, ki, qh, kh)
    np.testing.assert_array_equal(C.admissible_counts(qi, ki, qh, kh), mask.sum(axis=1))
    # brute force of the chunked scheme
    chunk = 32
    qo, ko = np.lexsort((qi, qh)), np.lexsort((ki, kh))
    seen = 0
    for s in range(T):
        lo, hi = max(0, chunk * (s // chunk - 1)), min(T, chunk * (s // chunk + 1))
        seen += sum(mask[qo[s], ko[t]] for t in range(lo, hi))
    assert C.chunked_coverage(qi, ki, qh, kh, chunk) == pytest.approx(seen / mask.sum())
    # a chunk covering everything sees every collision
    assert C.chunked_coverage(qi, ki, qh, kh, T) == 1.0


def test_chunked_coverage_falls_below_scfa_on_the_hash_workloads(capsys):
    w = WORKLOADS[2]  # 8192 tokens, 16 buckets
    rows = []
    for nb in (8, 16, 64):
        import dataclasses

        wn = dataclasses.replace(w, n_buckets=nb)
        hi = head_inputs(wn, 0, 0)
        R = lsh_rotation(wn, 0)
        qh, kh = lsh.buckets_c(hi.q, R), lsh.buckets_c(hi.k, R)
        covs = [C.chunked_coverage(hi.q_pos, hi.k_pos, qh, kh, c) for c in (64, 256)]
        rows.append((nb, *covs))
        assert all(0.0 < c < 1.0 for c in covs)
    with capsys.disabled():
        print("\ncoverage of admissible pairs (T=8192, one head): SCFA 1.000 by construction")
        for nb, c64, c256 in rows:
            print(f"  nb={nb:3d}: chunked c=64 {c64:.3f}, c=256 {c256:.3f}")
