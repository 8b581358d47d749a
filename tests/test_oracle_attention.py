"""Pins of the float64 attention oracle against things other than itself.

* causal reduction: identity positions and one bucket give standard causal
  attention (torch scaled_dot_product_attention, float64, and its autograd);
* QK-sparse with one shared ascending keep-set equals causal attention on
  the compacted tensors;
* Hash-sparse equals a per-bucket decomposition, each bucket run through
  torch's attention with an explicit boolean mask;
* closed forms with Q = 0 (uniform attention over admissible keys);
* invariants: rows of P sum to one (V = 1), gradient sums, permutation
  invariance, empty rows;
* gradients against central finite differences.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as A


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa(q, k, v, causal=False, mask=None, scale=None):
    tq = torch.from_numpy(np.ascontiguousarray(q))[None, None]
    tk = torch.from_numpy(np.ascontiguousarray(k))[None, None]
    tv = torch.from_numpy(np.ascontiguousarray(v))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal, scale=scale)[0, 0].numpy()


@pytest.mark.parametrize("T,d", [(1, 8), (37, 16), (130, 64)])
def test_identity_positions_single_bucket_is_causal_attention(T, d):
    rng = np.random.default_rng(T + d)
    q, k, v = _rand(rng, T, d), _rand(rng, T, d), _rand(rng, T, d)
    pos = np.arange(T)
    ref = _sdpa(q, k, v, causal=True)
    o_qk, _ = A.forward(q, k, v, pos, pos)
    zeros = np.zeros(T, dtype=np.int32)
    o_h, _ = A.forward(q, k, v, pos, pos, zeros, zeros)
    np.testing.assert_allclose(o_qk, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o_h, ref, rtol=0, atol=1e-12)


def test_identity_positions_gradients_match_autograd():
    rng = np.random.default_rng(7)
    T, d = 45, 16
    q, k, v, do = (_rand(rng, T, d) for _ in range(4))
    pos = np.arange(T)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    out = F.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None], is_causal=True)[0, 0]
    out.backward(torch.from_numpy(do))
    dq, dk, dv = A.backward(q, k, v, do, pos, pos)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11, rtol=0)


def test_shared_keep_set_equals_causal_attention_on_compacted_tensors():
    rng = np.random.default_rng(11)
    T, n, d = 300, 190, 32
    keep = np.sort(rng.choice(T, n, replace=False))
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o, _ = A.forward(q, k, v, keep, keep)
    np.testing.assert_allclose(o, _sdpa(q, k, v, causal=True), atol=1e-12, rtol=0)


def _bucket_decomposition(q, k, v, qi, ki, qh, kh, scale):
    """Within-bucket attention assembled bucket by bucket with torch's SDPA."""
    out = np.zeros((q.shape[0], v.shape[1]))
    for c in np.union1d(qh, kh):
        rq = np.nonzero(qh == c)[0]
        rk = np.nonzero(kh == c)[0]
        if len(rq) == 0 or len(rk) == 0:
            continue
        mask = ki[rk][None, :] <= qi[rq][:, None]
        has = mask.any(axis=1)
        if not has.any():
            continue
        o = _sdpa(q[rq][has], k[rk], v[rk], mask=mask[has], scale=scale)
        out[rq[has]] = o
    return out


@pytest.mark.parametrize("seed,nb", [(0, 2), (1, 5), (2, 16)])
def test_hash_mode_equals_per_bucket_decomposition(seed, nb):
    rng = np.random.default_rng(100 + seed)
    Tq, Tk, d = 150, 170, 16
    qi = np.sort(rng.choice(400, Tq, replace=False))
    ki = np.sort(rng.choice(400, Tk, replace=False))
    qh = rng.integers(0, nb, Tq)
    kh = rng.integers(0, nb, Tk)
    q, k, v = _rand(rng, Tq, d), _rand(rng, Tk, d), _rand(rng, Tk, d)
    # shuffle rows: the definition depends on positions, not on storage order
    pq, pk = rng.permutation(Tq), rng.permutation(Tk)
    q, qi, qh = q[pq], qi[pq], qh[pq]
    k, v, ki, kh = k[pk], v[pk], ki[pk], kh[pk]
    scale = 0.3
    o, lse = A.forward(q, k, v, qi, ki, qh, kh, scale)
    ref = _bucket_decomposition(q, k, v, qi, ki, qh, kh, scale)
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)
    empty = ~A.element_mask(qi, ki, qh, kh).any(axis=1)
    assert np.all(np.isneginf(lse[empty])) and np.all(np.isfinite(lse[~empty]))
    assert np.all(o[empty] == 0.0)


def test_zero_queries_closed_form():
    """Q = 0: every admissible score is 0, so lse_i = ln N_i and O_i = mean of admissible V."""
    rng = np.random.default_rng(5)
    Tq = Tk = 200
    qi = ki = np.arange(Tk)
    qh = rng.integers(0, 4, Tq)
    kh = rng.integers(0, 4, Tk)
    v = rng.integers(0, 2, (Tk, 3)).astype(np.float64)
    o, lse = A.forward(np.zeros((Tq, 8)), np.ones((Tk, 8)), v, qi, ki, qh, kh)
    for i in range(Tq):
        adm = [j for j in range(Tk) if ki[j] <= qi[i] and kh[j] == qh[i]]
        if not adm:
            assert np.isneginf(lse[i]) and np.all(o[i] == 0)
            continue
        assert lse[i] == pytest.approx(np.log(len(adm)), abs=1e-13)
        np.testing.assert_allclose(o[i], v[adm].mean(axis=0), atol=1e-14)


@pytest.mark.parametrize("shuffle", [False, True])
def test_zero_query_closed_form_all_rows(shuffle):
    """The O(T log T) Q = 0 evaluator equals the dense oracle and a brute-force loop."""
    rng = np.random.default_rng(11)
    Tq, Tk = 150, 170
    qi = np.sort(rng.choice(400, Tq, replace=False))
    ki = np.sort(rng.choice(400, Tk, replace=False))
    qh = rng.integers(0, 5, Tq)
    kh = rng.integers(0, 5, Tk)
    if shuffle:
        pq, pk = rng.permutation(Tq), rng.permutation(Tk)
        qi, qh, ki, kh = qi[pq], qh[pq], ki[pk], kh[pk]
    v = rng.integers(0, 2, (Tk, 4)).astype(np.float64)
    o, lse = A.zero_query_forward(qi, ki, v, qh, kh)
    o_ref, lse_ref = A.forward(np.zeros((Tq, 8)), rng.standard_normal((Tk, 8)), v, qi, ki, qh, kh)
    np.testing.assert_allclose(o, o_ref, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-13)
    for i in range(0, Tq, 7):
        adm = [j for j in range(Tk) if ki[j] <= qi[i] and kh[j] == qh[i]]
        if not adm:
            assert np.isneginf(lse[i]) and np.all(o[i] == 0)
        else:
            assert lse[i] == pytest.approx(np.log(len(adm)), abs=1e-13)
            np.testing.assert_allclose(o[i], v[adm].mean(axis=0), atol=1e-14)
    # QK mode (no buckets)
    o2, lse2 = A.zero_query_forward(qi, ki, v)
    o2_ref, lse2_ref = A.forward(np.zeros((Tq, 8)), rng.standard_normal((Tk, 8)), v, qi, ki)
    np.testing.assert_allclose(o2, o2_ref, atol=1e-13)
    np.testing.assert_allclose(lse2, lse2_ref, atol=1e-13)


def test_rows_of_p_sum_to_one():
    rng = np.random.default_rng(9)
    Tq, Tk, d = 90, 120, 8
    qi = rng.integers(0, 150, Tq)
    ki = rng.integers(0, 150, Tk)
    qh, kh = rng.integers(0, 3, Tq), rng.integers(0, 3, Tk)
    o, _ = A.forward(_rand(rng, Tq, d), _rand(rng, Tk, d), np.ones((Tk, 2)), qi, ki, qh, kh)
    nonempty = A.element_mask(qi, ki, qh, kh).any(axis=1)
    np.testing.assert_allclose(o[nonempty], 1.0, atol=1e-14)
    assert np.all(o[~nonempty] == 0.0)


def test_gradient_invariants():
    """sum_j dV_j = sum over non-empty rows of dO; sum_j dK_j = 0 (softmax shift invariance)."""
    rng = np.random.default_rng(21)
    Tq, Tk, d = 70, 80, 8
    qi, ki = rng.integers(0, 100, Tq), rng.integers(0, 100, Tk)
    qh, kh = rng.integers(0, 3, Tq), rng.integers(0, 3, Tk)
    q, k, v, do = _rand(rng, Tq, d), _rand(rng, Tk, d), _rand(rng, Tk, d), _rand(rng, Tq, d)
    dq, dk, dv = A.backward(q, k, v, do, qi, ki, qh, kh)
    nonempty = A.element_mask(qi, ki, qh, kh).any(axis=1)
    np.testing.assert_allclose(dv.sum(axis=0), do[nonempty].sum(axis=0), atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    assert np.all(dq[~nonempty] == 0.0)


def test_permutation_invariance():
    rng = np.random.default_rng(33)
    Tq, Tk, d = 60, 75, 8
    qi, ki = rng.integers(0, 90, Tq), rng.integers(0, 90, Tk)
    qh, kh = rng.integers(0, 4, Tq), rng.integers(0, 4, Tk)
    q, k, v, do = _rand(rng, Tq, d), _rand(rng, Tk, d), _rand(rng, Tk, d), _rand(rng, Tq, d)
    o, lse = A.forward(q, k, v, qi, ki, qh, kh)
    g = A.backward(q, k, v, do, qi, ki, qh, kh)
    pq, pk = rng.permutation(Tq), rng.permutation(Tk)
    o2, lse2 = A.forward(q[pq], k[pk], v[pk], qi[pq], ki[pk], qh[pq], kh[pk])
    np.testing.assert_allclose(o2, o[pq], atol=1e-13)
    np.testing.assert_allclose(lse2, lse[pq], atol=1e-13)
    g2 = A.backward(q[pq], k[pk], v[pk], do[pq], qi[pq], ki[pk], qh[pq], kh[pk])
    np.testing.assert_allclose(g2[0], g[0][pq], atol=1e-12)
    np.testing.assert_allclose(g2[1], g[1][pk], atol=1e-12)
    np.testing.assert_allclose(g2[2], g[2][pk], atol=1e-12)


@pytest.mark.parametrize("hashed", [False, True])
def test_gradients_match_central_finite_differences(hashed):
    rng = np.random.default_rng(3 + hashed)
    Tq, Tk, d = 9, 11, 5
    qi, ki = rng.integers(0, 12, Tq), rng.integers(0, 12, Tk)
    qh = rng.integers(0, 2, Tq) if hashed else None
    kh = rng.integers(0, 2, Tk) if hashed else None
    q, k, v, g = _rand(rng, Tq, d), _rand(rng, Tk, d), _rand(rng, Tk, d), _rand(rng, Tq, d)
    scale = 0.7

    def loss(qq, kk, vv):
        o, _ = A.forward(qq, kk, vv, qi, ki, qh, kh, scale)
        return float((o * g).sum())

    dq, dk, dv = A.backward(q, k, v, g, qi, ki, qh, kh, scale)
    h = 1e-6
    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.abs(num - grad).max() / max(1.0, np.abs(grad).max())
        assert err < 1e-6, (which, err)


def test_row_and_key_samplers_match_full_evaluation():
    rng = np.random.default_rng(44)
    Tq, Tk, d = 130, 140, 8
    qi, ki = np.sort(rng.choice(300, Tq, replace=False)), np.sort(rng.choice(300, Tk, replace=False))
    qh, kh = rng.integers(0, 3, Tq), rng.integers(0, 3, Tk)
    q, k, v, do = _rand(rng, Tq, d), _rand(rng, Tk, d), _rand(rng, Tk, d), _rand(rng, Tq, d)
    o, lse = A.forward(q, k, v, qi, ki, qh, kh)
    dq, dk, dv = A.backward(q, k, v, do, qi, ki, qh, kh)
    rows = [0, 5, 77, 129]
    o_r, lse_r = A.forward_rows(rows, q, k, v, qi, ki, qh, kh)
    np.testing.assert_array_equal(o_r, o[rows])
    np.testing.assert_array_equal(lse_r, lse[rows])
    np.testing.assert_allclose(A.backward_rows(rows, q, k, v, do, qi, ki, qh, kh), dq[rows], atol=1e-13)
    keys = [1, 60, 139]
    dk_r, dv_r = A.backward_key_rows(keys, q, k, v, do, qi, ki, qh, kh)
    np.testing.assert_allclose(dk_r, dk[keys], atol=1e-12)
    np.testing.assert_allclose(dv_r, dv[keys], atol=1e-12)


def test_chunking_does_not_change_results(monkeypatch):
    rng = np.random.default_rng(55)
    Tq, Tk, d = 100, 90, 8
    qi, ki = rng.integers(0, 120, Tq), rng.integers(0, 120, Tk)
    q, k, v, do = _rand(rng, Tq, d), _rand(rng, Tk, d), _rand(rng, Tk, d), _rand(rng, Tq, d)
    o, lse = A.forward(q, k, v, qi, ki)
    g = A.backward(q, k, v, do, qi, ki)
    monkeypatch.setattr(A, "_CHUNK", 7)
    o2, lse2 = A.forward(q, k, v, qi, ki)
    g2 = A.backward(q, k, v, do, qi, ki)
    np.testing.assert_allclose(o2, o, atol=1e-14)
    np.testing.assert_array_equal(lse2, lse)
    for a, b in zip(g, g2):
        np.testing.assert_allclose(a, b, atol=1e-13)
