"""Row gather / scatter on the GPU: bit-exact against the oracle, and the
whole path with them: compaction -> QK-sparse attention -> un-compaction,
and LSH sort -> Hash-sparse attention -> un-sort, against the oracle."""

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


def _t(a, dtype):
    return dev(a, torch.bfloat16 if dtype == "bf16" else torch.float32)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("fp32", 128), ("fp32", 4), ("bf16", 8)])
def test_gather_scatter_bit_exact(dtype, d):
    rng = np.random.default_rng(d)
    B, H, Ts, Td = 2, 3, 1000, 777
    src = rng.standard_normal((B, H, Ts, d)).astype(np.float32)
    if dtype == "bf16":
        src = bf16_round(src)
    idx = rng.integers(-5, Ts + 3, (B, H, Td)).astype(np.int32)  # some out of range
    note(f"[rows] gather {dtype} d={d}")
    g = to_np(_scfa().gather_rows(_t(src, dtype), dev(idx)))
    np.testing.assert_array_equal(g, Ro.gather_rows(src, idx))

    perm = np.stack([np.stack([rng.permutation(Ts) for _ in range(H)]) for _ in range(B)]).astype(np.int32)
    note(f"[rows] scatter perm {dtype} d={d}")
    s = to_np(_scfa().scatter_rows(_t(src, dtype), dev(perm), Ts))
    np.testing.assert_array_equal(s, Ro.scatter_rows(src, perm, Ts))

    # kept rows back to a longer sequence, with out-of-range rows dropped;
    # with and without zero fill
    T_full = 1500
    keep = np.stack([np.stack([np.sort(rng.choice(T_full, Ts, replace=False)) for _ in range(H)])
                     for _ in range(B)]).astype(np.int32)
    keep[0, 0, :3] = [-1, T_full, T_full + 9]
    base = np.full((B, H, T_full, d), 3.0, np.float32)
    note(f"[rows] scatter kept {dtype} d={d}")
    z = to_np(_scfa().scatter_rows(_t(src, dtype), dev(keep), T_full))
    np.testing.assert_array_equal(z, Ro.scatter_rows(src, keep, T_full))
    out = _t(base, dtype)
    nz = to_np(_scfa().scatter_rows(_t(src, dtype), dev(keep), T_full, zero_fill=False, out=out))
    np.testing.assert_array_equal(nz, Ro.scatter_rows(src, keep, T_full, zero_fill=False, base=base))


def test_empty_row_sets():
    scfa = _scfa()
    src = torch.ones((1, 2, 10, 64), dtype=torch.bfloat16, device="cuda:0")
    g = scfa.gather_rows(src, torch.zeros((1, 2, 0), dtype=torch.int32, device="cuda:0"))
    assert g.shape == (1, 2, 0, 64)
    s = scfa.scatter_rows(src[:, :, :0].contiguous(), torch.zeros((1, 2, 0), dtype=torch.int32, device="cuda:0"), 5)
    torch.cuda.synchronize()
    assert torch.count_nonzero(s).item() == 0


def test_compaction_attention_uncompaction():
    """Drop tokens, compact with gather, QK-sparse forward + backward on the
    compact tensors, scatter outputs and gradients back to the full length."""
    rng = np.random.default_rng(7)
    B, H, T, d, n_keep = 2, 3, 700, 64, 490
    full = [bf16_round(rng.standard_normal((B, H, T, d)).astype(np.float32)) for _ in range(4)]
    keep = np.stack([np.stack([np.sort(rng.choice(T, n_keep, replace=False)) for _ in range(H)])
                     for _ in range(B)]).astype(np.int32)
    scfa = _scfa()
    kd = dev(keep)
    note("[rows] compaction pipeline")
    q, k, v, do = (scfa.gather_rows(dev(x, torch.bfloat16), kd) for x in full)
    o, lse = scfa.qk_sparse_fwd(q, k, v, kd, kd)
    dq, dk, dv = scfa.qk_sparse_bwd(q, k, v, o, lse, do, kd, kd)
    O, dQ, dK, dV = (to_np(scfa.scatter_rows(x, kd, T)) for x in (o, dq, dk, dv))
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(d)
    for b in range(B):
        for h in range(H):
            qi = keep[b, h]
            Qc, Kc, Vc, Gc = (x[b, h][qi] for x in full)
            o_ref, lse_ref = A.forward(Qc, Kc, Vc, qi, qi, scale=scale)
            ref = A.backward(Qc, Kc, Vc, Gc, qi, qi, scale=scale)
            mask = np.zeros(T, bool)
            mask[qi] = True
            check_forward(O[b, h][qi], to_np(lse)[b, h], o_ref, lse_ref, "bf16", f"compaction b{b}h{h}")
            check_grads([dQ[b, h][qi], dK[b, h][qi], dV[b, h][qi]], ref, "bf16", f"compaction b{b}h{h}")
            for x in (O, dQ, dK, dV):
                assert np.all(x[b, h][~mask] == 0)


def test_hash_sort_attention_unsort():
    """LSH sort (rows gathered by the sort), Hash-sparse forward, un-sort with scatter."""
    rng = np.random.default_rng(8)
    B, H, T, d, nb = 1, 2, 900, 64, 8
    Q, K, V = (bf16_round(rng.standard_normal((B, H, T, d)).astype(np.float32)) for _ in range(3))
    R = rng.standard_normal((H, d, nb // 2)).astype(np.float32)
    scfa = _scfa()
    note("[rows] sort / un-sort pipeline")
    Rt = dev(R)
    qh, qi, qperm, qs, _ = scfa.lsh_bucket_sort(dev(Q, torch.bfloat16), Rt, nb)
    kh, ki, kperm, ks, vs = scfa.lsh_bucket_sort(dev(K, torch.bfloat16), Rt, nb, companion=dev(V, torch.bfloat16))
    o, lse = scfa.hash_sparse_fwd(qs, ks, vs, qi, ki, qh, kh)
    O = to_np(scfa.scatter_rows(o, qperm, T))
    torch.cuda.synchronize()
    pos = np.arange(T)
    for h in range(H):
        pq, hq, iq = lsh.bucket_sort(lsh.buckets(Q[0, h], R[h]), pos)
        pk, hk, ik = lsh.bucket_sort(lsh.buckets(K[0, h], R[h]), pos)
        o_ref, _ = A.forward(Q[0, h][pq], K[0, h][pk], V[0, h][pk], iq, ik, hq, hk, 1.0 / np.sqrt(d))
        o_orig = Ro.scatter_rows(o_ref[None, None], pq[None, None], T)[0, 0]
        check_forward(O[0, h], np.zeros(T), o_orig, np.zeros(T), "bf16", f"unsort h{h}")
