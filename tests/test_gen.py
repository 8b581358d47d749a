"""The seeded input generators: determinism, shapes, keep counts, bf16 exactness."""

import numpy as np
import torch

from gen import WORKLOADS, bf16_round, custom_workload, head_inputs, keep_set, lsh_rotation


def test_keep_counts():
    assert WORKLOADS[1].Tq == 179
    assert WORKLOADS[3].Tq == 5734
    assert WORKLOADS[5].Tq == 524288
    assert WORKLOADS[2].Tq == WORKLOADS[2].T == 8192


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000, dtype=np.float32) * np.float32(3.0)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(bf16_round(x), ref)
    np.testing.assert_array_equal(bf16_round(bf16_round(x)), bf16_round(x))


def test_deterministic_and_per_head():
    w = WORKLOADS[3]
    a = head_inputs(w, 1, 5)
    b = head_inputs(w, 1, 5)
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.q_pos, b.q_pos)
    c = head_inputs(w, 1, 6)
    assert not np.array_equal(a.q, c.q)
    assert a.do is not None and a.q.shape == (5734, 64)
    assert np.all(np.diff(a.q_pos) > 0) and a.q_pos is a.k_pos


def test_workload1_is_fp32_and_rotation_shapes():
    h = head_inputs(WORKLOADS[1], 0, 0)
    assert h.q.dtype == np.float32 and h.q.shape == (179, 64)
    assert not np.array_equal(bf16_round(h.q), h.q)
    assert lsh_rotation(WORKLOADS[4], 3).shape == (64, 16)
    assert lsh_rotation(WORKLOADS[5], 0).shape == (128, 128)


def test_independent_keep_sets():
    w = custom_workload(seed=9, mode="qk", T=500, n_keep=300, n_keep_k=200)
    q, k = keep_set(w, 0, 0)
    assert q.shape == (300,) and k.shape == (200,)
    assert np.all(np.diff(q) > 0) and np.all(np.diff(k) > 0)
