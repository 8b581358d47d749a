"""The five benchmark workloads at full size, end to end on the GPU.

Hash workloads run the whole path on the GPU: LSH bucket ids and the
(bucket, position) sort of Q (with dO) and of K (with V), block metadata,
forward and backward.  The CPU oracle recomputes every bucket id, permutation
and position bit-exactly, then the attention outputs in float64: densely for
the smaller workloads and a subset of heads, and on sampled rows (each exact
against every key of its head) everywhere else.
"""

import numpy as np
import pytest

from gen import WORKLOADS, head_inputs, lsh_rotation
from helpers import check_forward, check_grads, dev, note, rel_fro, to_np
from oracle import attention as A
from oracle import lsh

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _scfa():
    import sparse_causal_attention_amd as scfa

    return scfa


def _stack(w):
    heads = [[head_inputs(w, b, h) for h in range(w.H)] for b in range(w.B)]
    st = lambda f: np.stack([np.stack([f(x) for x in row]) for row in heads])  # noqa: E731
    Q, K, V = st(lambda x: x.q), st(lambda x: x.k), st(lambda x: x.v)
    dO = st(lambda x: x.do) if w.train else None
    return Q, K, V, dO, st(lambda x: x.q_pos), st(lambda x: x.k_pos)


def _rows_sample(rng, T, n):
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, min(n, T), replace=False)]))


def test_workload1_qk_fwd_fp32():
    w = WORKLOADS[1]
    Q, K, V, _, qp, kp = _stack(w)
    do = np.random.default_rng(1).standard_normal(Q.shape).astype(np.float32)
    note(f"[workload] {w.name}")
    scfa = _scfa()
    q, k, v = dev(Q), dev(K), dev(V)
    qi, ki = dev(qp), dev(kp)
    o, lse = scfa.qk_sparse_fwd(q, k, v, qi, ki, block=w.block, scale=w.scale)
    grads = scfa.qk_sparse_bwd(q, k, v, o, lse, dev(do), qi, ki, block=w.block, scale=w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.forward(Q[0, 0], K[0, 0], V[0, 0], qp[0, 0], kp[0, 0], scale=w.scale)
    check_forward(to_np(o)[0, 0], to_np(lse)[0, 0], o_ref, lse_ref, "fp32", w.name)
    ref = A.backward(Q[0, 0], K[0, 0], V[0, 0], do[0, 0], qp[0, 0], kp[0, 0], scale=w.scale)
    check_grads([to_np(g)[0, 0] for g in grads], ref, "fp32", w.name)


def test_workload3_qk_train_bf16():
    w = WORKLOADS[3]
    Q, K, V, dO, qp, kp = _stack(w)
    note(f"[workload] {w.name}")
    scfa = _scfa()
    q, k, v, do = (dev(a, torch.bfloat16) for a in (Q, K, V, dO))
    qi, ki = dev(qp), dev(kp)
    o, lse = scfa.qk_sparse_fwd(q, k, v, qi, ki, block=w.block, scale=w.scale)
    dq, dk, dv = scfa.qk_sparse_bwd(q, k, v, o, lse, do, qi, ki, block=w.block, scale=w.scale)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (to_np(t) for t in (o, lse, dq, dk, dv))
    rng = np.random.default_rng(3)
    # full dense oracle on a few heads
    for b, h in [(0, 0), (1, 5), (3, 11)]:
        o_ref, lse_ref = A.forward(Q[b, h], K[b, h], V[b, h], qp[b, h], kp[b, h], scale=w.scale)
        check_forward(o[b, h], lse[b, h], o_ref, lse_ref, "bf16", f"{w.name} b{b}h{h}")
        ref = A.backward(Q[b, h], K[b, h], V[b, h], dO[b, h], qp[b, h], kp[b, h], scale=w.scale)
        check_grads([dq[b, h], dk[b, h], dv[b, h]], ref, "bf16", f"{w.name} b{b}h{h}")
    # sampled rows on every head
    for b in range(w.B):
        for h in range(w.H):
            rows = _rows_sample(rng, w.Tq, 48)
            o_ref, lse_ref = A.forward_rows(rows, Q[b, h], K[b, h], V[b, h], qp[b, h], kp[b, h], scale=w.scale)
            check_forward(o[b, h][rows], lse[b, h][rows], o_ref, lse_ref, "bf16", f"{w.name} rows b{b}h{h}")
            dq_ref = A.backward_rows(rows, Q[b, h], K[b, h], V[b, h], dO[b, h], qp[b, h], kp[b, h], scale=w.scale)
            assert rel_fro(dq[b, h][rows], dq_ref) <= 5e-2
    _zero_query_all_rows(w, {(b, h): (qp[b, h], kp[b, h], None, None) for b in range(w.B) for h in range(w.H)})


def _hash_pipeline(w, Q, K, V, dO, qp, kp):
    """Whole GPU path; returns sorted outputs and the GPU's sort results."""
    scfa = _scfa()
    R = np.stack([lsh_rotation(w, h) for h in range(w.H)])
    q, k, v = (dev(a, torch.bfloat16) for a in (Q, K, V))
    do = dev(dO, torch.bfloat16) if dO is not None else None
    Rt = dev(R)
    pos_q = None if w.mode == "hash" else dev(qp)
    pos_k = None if w.mode == "hash" else dev(kp)
    qh, qi, qperm, qs, dos = scfa.lsh_bucket_sort(q, Rt, w.n_buckets, idx=pos_q, companion=do, idx_ascending=True)
    del q
    kh, ki, kperm, ks, vs = scfa.lsh_bucket_sort(k, Rt, w.n_buckets, idx=pos_k, companion=v, idx_ascending=True)
    del k, v
    o, lse = scfa.hash_sparse_fwd(qs, ks, vs, qi, ki, qh, kh, block=w.block, scale=w.scale)
    grads = None
    if w.train:
        grads = scfa.hash_sparse_bwd(qs, ks, vs, o, lse, dos, qi, ki, qh, kh, block=w.block, scale=w.scale)
    torch.cuda.synchronize()
    return R, dict(qh=qh, qi=qi, qperm=qperm, kh=kh, ki=ki, kperm=kperm), o, lse, grads


def _check_sort(R, srt, X, pos, b, h, which):
    bk = lsh.buckets_c(X[b, h], R[h])
    p_ref, h_ref, i_ref = lsh.bucket_sort(bk, pos[b, h])
    np.testing.assert_array_equal(srt[which + "perm"][b, h].cpu().numpy(), p_ref)
    np.testing.assert_array_equal(srt[which + "h"][b, h].cpu().numpy(), h_ref)
    np.testing.assert_array_equal(srt[which + "i"][b, h].cpu().numpy(), i_ref)
    return p_ref, h_ref, i_ref


def _zero_query_all_rows(w, heads):
    """Closed form at full size: Q = 0 makes P uniform over the admissible keys.

    ``heads`` maps (b, h) to the oracle's (q_idx, k_idx, q_hash, k_hash); the
    bucket ids are None in QK-sparse mode.
    K is 0 as well (scores are 0 whatever K is) and V holds binary features
    of each key's position and bucket, exact in bf16, so O_i is the mean of
    the admissible keys' features: every row of every head is compared with
    the oracle's O(T log T) evaluation, within bf16 rounding of a value in
    [0, 1] (2^-9) for O and float32 log for lse.
    """
    scfa = _scfa()
    B, H, Tq, Tk, d = w.B, w.H, w.Tq, w.Tk, w.d
    bits = np.arange(d)

    hashed = w.mode != "qk"

    def feats(ki, kh):
        kh = ki * 7 if kh is None else kh
        f = np.where(bits < d // 2, (ki[:, None] >> (bits % 20)) & 1, (kh[:, None] >> (bits % 8)) & 1)
        return f.astype(np.float32)

    stack = lambda i: np.stack([np.stack([heads[(b, h)][i] for h in range(H)]) for b in range(B)])  # noqa: E731
    iq, ik = (dev(stack(i).astype(np.int32)) for i in range(2))
    hq, hk = (dev(stack(i).astype(np.int32)) for i in (2, 3)) if hashed else (None, None)
    v = torch.empty((B, H, Tk, d), dtype=torch.bfloat16, device="cuda:0")
    for (b, h), (_, ki, _, kh) in heads.items():
        v[b, h] = torch.from_numpy(feats(ki, kh)).to(torch.bfloat16)
    zq = torch.zeros((B, H, Tq, d), dtype=torch.bfloat16, device="cuda:0")
    zk = torch.zeros((B, H, Tk, d), dtype=torch.bfloat16, device="cuda:0")
    note(f"[workload] {w.name}: Q = 0 closed form on all {B * H * Tq} rows")
    if hashed:
        o, lse = scfa.hash_sparse_fwd(zq, zk, v, iq, ik, hq, hk, block=w.block, scale=w.scale)
    else:
        o, lse = scfa.qk_sparse_fwd(zq, zk, v, iq, ik, block=w.block, scale=w.scale)
    torch.cuda.synchronize()
    del zq, zk, v
    for (b, h), (qi, ki, qh, kh) in heads.items():
        o_ref, lse_ref = A.zero_query_forward(qi, ki, feats(ki, kh).astype(np.float64), qh, kh)
        og = o[b, h].float().cpu().numpy()
        lg = lse[b, h].cpu().numpy()
        empty = np.isneginf(lse_ref)
        assert np.array_equal(np.isneginf(lg), empty), f"b{b}h{h}: empty rows differ"
        assert np.all(og[empty] == 0)
        np.testing.assert_allclose(og, o_ref, rtol=0, atol=2.0 ** -9 + 1e-6, err_msg=f"O b{b}h{h}")
        np.testing.assert_allclose(lg[~empty], lse_ref[~empty], rtol=0, atol=1e-5, err_msg=f"lse b{b}h{h}")


@pytest.mark.parametrize("wid", [2, 4])
def test_hash_workloads(wid):
    w = WORKLOADS[wid]
    Q, K, V, dO, qp, kp = _stack(w)
    note(f"[workload] {w.name}")
    R, srt, o, lse, grads = _hash_pipeline(w, Q, K, V, dO, qp, kp)
    o, lse = to_np(o), to_np(lse)
    g = [to_np(t) for t in grads] if grads is not None else None
    rng = np.random.default_rng(wid)
    full_heads = {(0, 0), (w.B - 1, w.H - 1)} if wid == 4 else {(0, h) for h in range(w.H)}
    sorted_heads = {}
    for b in range(w.B):
        for h in range(w.H):
            pq, hq, iq = _check_sort(R, srt, Q, qp, b, h, "q")
            pk, hk, ik = _check_sort(R, srt, K, kp, b, h, "k")
            sorted_heads[(b, h)] = (iq, ik, hq, hk)
            qs, ks, vs = Q[b, h][pq], K[b, h][pk], V[b, h][pk]
            if (b, h) in full_heads:
                o_ref, lse_ref = A.forward(qs, ks, vs, iq, ik, hq, hk, w.scale)
                check_forward(o[b, h], lse[b, h], o_ref, lse_ref, "bf16", f"{w.name} b{b}h{h}")
                if g is not None:
                    ref = A.backward(qs, ks, vs, dO[b, h][pq], iq, ik, hq, hk, w.scale)
                    check_grads([g[0][b, h], g[1][b, h], g[2][b, h]], ref, "bf16", f"{w.name} b{b}h{h}")
            else:
                rows = _rows_sample(rng, w.Tq, 64)
                o_ref, lse_ref = A.forward_rows(rows, qs, ks, vs, iq, ik, hq, hk, w.scale)
                check_forward(o[b, h][rows], lse[b, h][rows], o_ref, lse_ref, "bf16", f"{w.name} rows b{b}h{h}")
                if g is not None:
                    dq_ref = A.backward_rows(rows, qs, ks, vs, dO[b, h][pq], iq, ik, hq, hk, w.scale)
                    assert rel_fro(g[0][b, h][rows], dq_ref) <= 5e-2
                    keys = _rows_sample(rng, w.Tk, 16)
                    dk_ref, dv_ref = A.backward_key_rows(keys, qs, ks, vs, dO[b, h][pq], iq, ik, hq, hk, w.scale)
                    assert rel_fro(g[1][b, h][keys], dk_ref) <= 5e-2
                    assert rel_fro(g[2][b, h][keys], dv_ref) <= 5e-2
    del o, lse, g, srt
    _zero_query_all_rows(w, sorted_heads)


def test_workload5_million_token_hash_drop():
    w = WORKLOADS[5]
    note(f"[workload] {w.name}")
    Q, K, V, _, qp, kp = _stack(w)
    R, srt, o, lse, _ = _hash_pipeline(w, Q, K, V, None, qp, kp)
    o, lse = to_np(o), to_np(lse)
    rng = np.random.default_rng(5)
    sorted_heads = {}
    for h in range(w.H):
        pq, hq, iq = _check_sort(R, srt, Q, qp, 0, h, "q")
        pk, hk, ik = _check_sort(R, srt, K, kp, 0, h, "k")
        sorted_heads[(0, h)] = (iq, ik, hq, hk)
        rows = _rows_sample(rng, w.Tq, 64)
        o_ref, lse_ref = A.forward_rows(rows, Q[0, h][pq], K[0, h][pk], V[0, h][pk], iq, ik, hq, hk, w.scale)
        check_forward(o[0, h][rows], lse[0, h][rows], o_ref, lse_ref, "bf16", f"{w.name} rows h{h}")
    del Q, K, V, o, lse, srt
    _zero_query_all_rows(w, sorted_heads)
