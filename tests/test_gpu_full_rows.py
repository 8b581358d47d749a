"""Attention and the LSH sort over the kept rows of full-length tensors, read in place.

Dropping tokens keeps each kept token's original position ("1. QK-Sparse"), so the kept rows need not
be copied into compact tensors.
* Q, K, V (and dO) stay full length. q_rows / k_rows hold the kept positions, with Tq_src / Tk_src set
  to the full length. FLAG_ORIG_ROWS writes every output at its token's original row.
* zero_rows clears the rows of the dropped tokens.
* The LSH sort reads the kept rows through x_rows.

Every result must equal the compaction pipeline bit for bit:
gather -> LSH / attention over the compact tensors -> scatter with zero fill.
One head of each case is also checked against the oracle.
"""

import numpy as np
import pytest

from gen import bf16_round
from helpers import check_forward, check_grads, dev, note, to_np
from oracle import attention as A
from oracle import lsh
from oracle import rows as Ro

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _scfa():
    import sparse_causal_attention_amd as scfa

    return scfa


def _keep_drop(rng, B, H, T, n):
    keep = np.stack([np.stack([np.sort(rng.choice(T, n, replace=False)) for _ in range(H)]) for _ in range(B)])
    drop = np.stack([np.stack([np.setdiff1d(np.arange(T), keep[b, h]) for h in range(H)]) for b in range(B)])
    return keep.astype(np.int32), drop.astype(np.int32)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("fp32", 128), ("bf16", 8)])
def test_zero_rows_bit_exact(dtype, d):
    rng = np.random.default_rng(40 + d)
    B, H, T, n = 2, 3, 800, 333
    dst = rng.standard_normal((B, H, T, d)).astype(np.float32)
    if dtype == "bf16":
        dst = bf16_round(dst)
    index = rng.integers(-4, T + 4, (B, H, n)).astype(np.int32)  # some out of range, some repeated
    t = dev(dst, torch.bfloat16 if dtype == "bf16" else torch.float32)
    note(f"[full rows] zero_rows {dtype} d={d}")
    out = _scfa().zero_rows(t, dev(index))
    torch.cuda.synchronize()
    assert out.data_ptr() == t.data_ptr()
    np.testing.assert_array_equal(to_np(out), Ro.zero_rows(dst, index))
    empty = _scfa().zero_rows(t, torch.zeros((B, H, 0), dtype=torch.int32, device="cuda:0"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(empty), Ro.zero_rows(dst, index))


@pytest.mark.parametrize("block,stored_ds", [(64, False), (64, True), (128, False)])
def test_qk_training_on_full_length_tensors(block, stored_ds):
    """QK-sparse forward and backward over the kept rows of full-length Q, K, V, dO (30 % dropped per
    head, a ragged last block) equal the compaction pipeline bit for bit; one head against the oracle."""
    rng = np.random.default_rng(17 + block)
    B, H, T, n, d = 2, 2, 900, 631, 64
    full = [bf16_round(rng.standard_normal((B, H, T, d)).astype(np.float32)) for _ in range(4)]
    keep, drop = _keep_drop(rng, B, H, T, n)
    scfa = _scfa()
    q, k, v, do = (dev(x, torch.bfloat16) for x in full)
    kd, dd = dev(keep), dev(drop)
    meta = scfa.block_meta(kd, kd, block=block, with_cols=True, exact=True)
    F = 1 << 4  # FLAG_ORIG_ROWS
    note(f"[full rows] qk training block={block} stored_ds={stored_ds}: compaction path")
    qc, kc, vc, dc = (scfa.gather_rows(x, kd) for x in (q, k, v, do))
    if stored_ds:
        scfa.tile_slots(meta)
        ds = scfa.ds_buffer(int(meta["col_base"][-1].item()), block)
    o1, l1 = scfa.attn_fwd_lists(qc, kc, vc, kd, kd, None, None, meta, block=block)
    if stored_ds:
        de1 = scfa.attn_bwd_prep(o1, l1, dc)
        dk1, dv1 = scfa.attn_bwd_dkdv_ds_lists(qc, kc, vc, l1, dc, de1, kd, kd, None, None, meta, ds, block=block)
        dq1 = scfa.attn_bwd_dq_ds_lists(qc, kc, vc, o1, l1, dc, kd, kd, None, None, meta, ds, de1, block=block)
    else:
        dq1, de1 = scfa.attn_bwd_dq_lists(qc, kc, vc, o1, l1, dc, kd, kd, None, None, meta, block=block)
        dk1, dv1 = scfa.attn_bwd_dkdv_lists(qc, kc, vc, l1, dc, de1, kd, kd, None, None, meta, block=block)
    ref = [scfa.scatter_rows(x, kd, T) for x in (o1, dq1, dk1, dv1)]

    note(f"[full rows] qk training block={block} stored_ds={stored_ds}: in place")
    rows = dict(q_rows=kd, k_rows=kd, flags=F, block=block)
    o2, l2 = scfa.attn_fwd_lists(q, k, v, kd, kd, None, None, meta, **rows)
    if stored_ds:
        de2 = scfa.attn_bwd_prep(o2, l2, do, q_rows=kd, flags=F)
        dk2, dv2 = scfa.attn_bwd_dkdv_ds_lists(q, k, v, l2, do, de2, kd, kd, None, None, meta, ds, **rows)
        dq2 = scfa.attn_bwd_dq_ds_lists(q, k, v, o2, l2, do, kd, kd, None, None, meta, ds, de2, **rows)
    else:
        dq2, de2 = scfa.attn_bwd_dq_lists(q, k, v, o2, l2, do, kd, kd, None, None, meta, **rows)
        dk2, dv2 = scfa.attn_bwd_dkdv_lists(q, k, v, l2, do, de2, kd, kd, None, None, meta, **rows)
    got = [scfa.zero_rows(x, dd) for x in (o2, dq2, dk2, dv2)]
    torch.cuda.synchronize()
    assert o2.shape == (B, H, T, d) and l2.shape == (B, H, T) and dk2.shape == (B, H, T, d)
    for name, a_, b_ in zip(("o", "dq", "dk", "dv"), ref, got):
        assert torch.equal(a_, b_), name
    assert torch.equal(de1, de2)
    assert torch.equal(torch.gather(l2, 2, kd.long()), l1)

    b, h = 1, 1
    qi = keep[b, h]
    Qc, Kc, Vc, Gc = (x[b, h][qi] for x in full)
    scale = 1.0 / np.sqrt(d)
    o_ref, lse_ref = A.forward(Qc, Kc, Vc, qi, qi, scale=scale)
    g_ref = A.backward(Qc, Kc, Vc, Gc, qi, qi, scale=scale)
    O, L, dQ, dK, dV = (to_np(x) for x in (got[0], l2, got[1], got[2], got[3]))
    check_forward(O[b, h][qi], L[b, h][qi], o_ref, lse_ref, "bf16", "full-length rows")
    check_grads([dQ[b, h][qi], dK[b, h][qi], dV[b, h][qi]], g_ref, "bf16", "full-length rows")
    for x in (O, dQ, dK, dV):
        assert np.all(x[b, h][drop[b, h]] == 0)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("fp32", 64)])
def test_lsh_sort_through_rows_equals_compacted(dtype, d):
    """The LSH sort reading the kept rows of a full-length x through x_rows gives the bucket ids,
    positions and permutation of the sort over the gathered compact x, bit for bit."""
    rng = np.random.default_rng(60 + d)
    B, H, T, n, nb = 2, 2, 1100, 700, 16
    x = rng.standard_normal((B, H, T, d)).astype(np.float32)
    if dtype == "bf16":
        x = bf16_round(x)
    R = rng.standard_normal((H, d, nb // 2)).astype(np.float32)
    keep, _ = _keep_drop(rng, B, H, T, n)
    rows, rows_ok = keep.copy(), keep.copy()
    rows[0, 1, 5], rows_ok[0, 1, 5] = -3, 0  # out of range: the device clamps it to row 0
    scfa = _scfa()
    tx = dev(x, torch.bfloat16 if dtype == "bf16" else torch.float32)
    kd, Rt = dev(keep), dev(R)
    note(f"[full rows] lsh through rows {dtype} d={d}")
    xc = scfa.gather_rows(tx, dev(rows_ok))
    a = scfa.lsh_bucket_sort(xc, Rt, nb, idx=kd, want_x=False)
    b_ = scfa.lsh_bucket_sort(tx, Rt, nb, idx=kd, want_x=False, x_rows=dev(rows))
    torch.cuda.synchronize()
    for u, w in zip(a[:3], b_[:3]):
        assert torch.equal(u, w)
    # one head against the oracle's buckets and (bucket, position) order
    hh, ii, pp = (to_np(t) for t in b_[:3])
    xr = x[1, 0][keep[1, 0]]
    perm, hs, ids = lsh.bucket_sort(lsh.buckets(xr, R[0]), keep[1, 0])
    np.testing.assert_array_equal(hh[1, 0], hs)
    np.testing.assert_array_equal(ii[1, 0], ids)
    np.testing.assert_array_equal(pp[1, 0], perm)


@pytest.mark.parametrize("d,block", [(64, 64), (128, 128)])
def test_hash_drop_forward_on_full_length_tensors(d, block):
    """50 % of the tokens dropped, then LSH over the kept rows of the stacked full-length Q and K
    (x_rows), lists, the Hash-sparse forward reading Q, K, V at the kept positions and writing O
    there, and the dropped rows cleared.  This equals the compaction pipeline bit for bit:
    gather -> LSH over the compact Q, K -> forward through the sort permutation -> scatter with zero
    fill.  One head is checked against the oracle."""
    rng = np.random.default_rng(80 + d)
    B, H, T, n, nb = 1, 2, 1400, 700, 8
    Q, K, V = (bf16_round(rng.standard_normal((B, H, T, d)).astype(np.float32)) for _ in range(3))
    R = rng.standard_normal((H, d, nb // 2)).astype(np.float32)
    keep, drop = _keep_drop(rng, B, H, T, n)
    scfa = _scfa()
    qk = dev(np.concatenate([Q, K]), torch.bfloat16)
    v = dev(V, torch.bfloat16)
    kd, dd, Rt = dev(keep), dev(drop), dev(R)
    keep2 = torch.cat([kd, kd]).contiguous()
    note(f"[full rows] hash drop forward d={d} block={block}: compaction path")
    qkc = scfa.gather_rows(qk, keep2)
    vc = scfa.gather_rows(v, kd)
    hh, ii, pp, _, _ = scfa.lsh_bucket_sort(qkc, Rt, nb, idx=keep2, idx_ascending=True, want_x=False)
    qh, kh, qi, ki = hh[:B], hh[B:], ii[:B], ii[B:]
    meta = scfa.block_meta(qi, ki, qh, kh, block=block, with_cols=False, exact=True)
    o1, l1 = scfa.attn_fwd_lists(qkc[:B], qkc[B:], vc, qi, ki, qh, kh, meta, block=block, q_rows=pp[:B],
                                 k_rows=pp[B:])
    O1 = scfa.scatter_rows(o1, qi, T)

    note(f"[full rows] hash drop forward d={d} block={block}: in place")
    hh2, ii2, pp2, _, _ = scfa.lsh_bucket_sort(qk, Rt, nb, idx=keep2, idx_ascending=True, want_x=False, x_rows=keep2)
    o2, l2 = scfa.attn_fwd_lists(qk[:B], qk[B:], v, ii2[:B], ii2[B:], hh2[:B], hh2[B:], meta, block=block,
                                 q_rows=ii2[:B], k_rows=ii2[B:], flags=1 << 4)
    O2 = scfa.zero_rows(o2, dd)
    torch.cuda.synchronize()
    for u, w in ((hh, hh2), (ii, ii2), (pp, pp2), (O1, O2)):
        assert torch.equal(u, w)
    assert torch.equal(torch.gather(l2, 2, qi.long()), l1)

    h = 1
    pos = keep[0, h]
    pq, hq, iq = lsh.bucket_sort(lsh.buckets(Q[0, h][pos], R[h]), pos)
    pk, hk, ik = lsh.bucket_sort(lsh.buckets(K[0, h][pos], R[h]), pos)
    o_ref, lse_ref = A.forward(Q[0, h][pos][pq], K[0, h][pos][pk], V[0, h][pos][pk], iq, ik, hq, hk, 1.0 / np.sqrt(d))
    O = to_np(O2)[0, h]
    check_forward(O[iq], to_np(l2)[0, h][iq], o_ref, lse_ref, "bf16", f"hash drop in place d={d}")
    assert np.all(O[drop[0, h]] == 0)


def test_independent_q_and_k_drops_from_tensors_of_different_lengths():
    """Q kept from a 900-row tensor, K and V from a 1000-row one, with independent kept sets (600 and 700
    rows): every row count differs (Tq, Tk, Tq_src, Tk_src), and the forward and both backward kernels in
    place equal the compaction pipeline bit for bit; outputs land at each side's own kept positions."""
    rng = np.random.default_rng(97)
    B, H, Tqf, Tkf, nq, nk, d = 2, 2, 900, 1000, 600, 700, 64
    qf, dof = (bf16_round(rng.standard_normal((B, H, Tqf, d)).astype(np.float32)) for _ in range(2))
    kf, vf = (bf16_round(rng.standard_normal((B, H, Tkf, d)).astype(np.float32)) for _ in range(2))
    kq, dq_drop = _keep_drop(rng, B, H, Tqf, nq)
    kk, dk_drop = _keep_drop(rng, B, H, Tkf, nk)
    scfa = _scfa()
    q, do = (dev(x, torch.bfloat16) for x in (qf, dof))
    k, v = (dev(x, torch.bfloat16) for x in (kf, vf))
    qi, ki, qdd, kdd = dev(kq), dev(kk), dev(dq_drop), dev(dk_drop)
    meta = scfa.block_meta(qi, ki, block=64, with_cols=True, exact=True)
    note("[full rows] independent drops: compaction path")
    qc, dc = scfa.gather_rows(q, qi), scfa.gather_rows(do, qi)
    kc, vc = scfa.gather_rows(k, ki), scfa.gather_rows(v, ki)
    o1, l1 = scfa.attn_fwd_lists(qc, kc, vc, qi, ki, None, None, meta)
    dq1, de1 = scfa.attn_bwd_dq_lists(qc, kc, vc, o1, l1, dc, qi, ki, None, None, meta)
    dk1, dv1 = scfa.attn_bwd_dkdv_lists(qc, kc, vc, l1, dc, de1, qi, ki, None, None, meta)
    ref = [scfa.scatter_rows(o1, qi, Tqf), scfa.scatter_rows(dq1, qi, Tqf), scfa.scatter_rows(dk1, ki, Tkf),
           scfa.scatter_rows(dv1, ki, Tkf)]
    note("[full rows] independent drops: in place")
    rows = dict(q_rows=qi, k_rows=ki, flags=1 << 4)
    o2, l2 = scfa.attn_fwd_lists(q, k, v, qi, ki, None, None, meta, **rows)
    dq2, de2 = scfa.attn_bwd_dq_lists(q, k, v, o2, l2, do, qi, ki, None, None, meta, **rows)
    dk2, dv2 = scfa.attn_bwd_dkdv_lists(q, k, v, l2, do, de2, qi, ki, None, None, meta, **rows)
    got = [scfa.zero_rows(o2, qdd), scfa.zero_rows(dq2, qdd), scfa.zero_rows(dk2, kdd), scfa.zero_rows(dv2, kdd)]
    torch.cuda.synchronize()
    assert o2.shape == (B, H, Tqf, d) and dk2.shape == (B, H, Tkf, d) and l2.shape == (B, H, Tqf)
    for name, a_, b_ in zip(("o", "dq", "dk", "dv"), ref, got):
        assert torch.equal(a_, b_), name
    assert torch.equal(de1, de2)
    assert torch.equal(torch.gather(l2, 2, qi.long()), l1)
    b, h = 0, 1
    Qc, Gc, Kc, Vc = qf[b, h][kq[b, h]], dof[b, h][kq[b, h]], kf[b, h][kk[b, h]], vf[b, h][kk[b, h]]
    o_ref, lse_ref = A.forward(Qc, Kc, Vc, kq[b, h], kk[b, h], scale=1.0 / np.sqrt(d))
    g_ref = A.backward(Qc, Kc, Vc, Gc, kq[b, h], kk[b, h], scale=1.0 / np.sqrt(d))
    O, L, dQ, dK, dV = (to_np(x) for x in (got[0], l2, got[1], got[2], got[3]))
    check_forward(O[b, h][kq[b, h]], L[b, h][kq[b, h]], o_ref, lse_ref, "bf16", "independent drops")
    check_grads([dQ[b, h][kq[b, h]], dK[b, h][kk[b, h]], dV[b, h][kk[b, h]]], g_ref, "bf16", "independent drops")
