"""The timed steps of the two dropped-token workloads, at full size, against the oracle.

``bench.workload_setup`` builds the inputs and the step exactly as the benchmark times them. No kept
row is copied in either step:
* QK-sparse training, 4 x 12 heads of 8,192 tokens with 30 % dropped per head. Lists, forward, dQ and
  dK/dV run over the kept rows of the full-length Q, K, V, dO, read in place. Outputs are written at
  the kept positions and the dropped rows are cleared.
* Hash-sparse forward after a 50 % drop: 8 heads of 1,048,576 tokens, d = 128, 256 buckets, block 128.
  LSH + sort runs over the kept rows of the stacked full-length Q and K. Then the lists, the forward
  reading and writing at the kept positions, and the dropped rows of O cleared.

The inputs are drawn on the GPU from a seeded generator and copied back head by head. The oracle
recomputes:
* the lists (QK-sparse) and the bucket ids and (bucket, position) order (Hash-sparse) bit for bit;
* O, lse and the gradients densely on full heads, and on sampled rows of the other heads;
* zero rows at every dropped position.
"""

import numpy as np
import pytest

from gen import WORKLOADS, keep_set, lsh_rotation
from helpers import check_forward, check_grads, note, rel_fro, to_np
from oracle import attention as A
from oracle import blocks as Bk
from oracle import lsh

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _rows_sample(rng, T, n):
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, min(n, T), replace=False)]))


def _head(t, b, h):
    return t[b, h].float().cpu().numpy()


@pytest.mark.timeout(600)
def test_workload3_step_matches_oracle():
    import bench
    import sparse_causal_attention_amd as scfa

    note("[workload step] qk_train_bf16_T8192_drop30: inputs and one step")
    w, step, _, dense_in = bench.workload_setup(scfa, torch, 3)
    assert w.name == "qk_train_bf16_T8192_drop30"
    meta, outs = step(None)
    torch.cuda.synchronize()
    q, k, v, do = dense_in
    got_lists = {n: meta[n].cpu().numpy() for n in ("row_count", "row_list", "col_count", "col_list")}
    rng = np.random.default_rng(8192)
    full_heads = {(0, 0), (w.B - 1, w.H - 1)}
    for b in range(w.B):
        for h in range(w.H):
            keep = keep_set(w, b, h)[0]
            mask = np.zeros(w.T, bool)
            mask[keep] = True
            Q, K, V, G = (_head(t, b, h) for t in (q, k, v, do))
            O, L, dQ, dK, dV = (_head(outs[n], b, h) for n in ("o", "lse", "dq", "dk", "dv"))
            for x in (O, dQ, dK, dV):
                assert np.all(x[~mask] == 0), (b, h)
            Qc, Kc, Vc, Gc = Q[keep], K[keep], V[keep], G[keep]
            o_v, lse_v, dq_v, dk_v, dv_v = O[keep], L[keep], dQ[keep], dK[keep], dV[keep]
            if (b, h) in full_heads:
                note(f"[workload step] qk full oracle b{b}h{h}")
                _, _, live, free = Bk.metadata_exact(keep, keep, None, None, w.block)
                for i, row in enumerate(Bk.row_lists(live, free)):
                    n = int(got_lists["row_count"][b, h, i])
                    want = [j | (0x80000000 if f else 0) for j, f in row]
                    assert list(got_lists["row_list"][b, h, i, :n].view(np.uint32)) == want, (b, h, i)
                for j, colv in enumerate(Bk.col_lists(live, free)):
                    n = int(got_lists["col_count"][b, h, j])
                    want = [i | (0x80000000 if f else 0) for i, f in colv]
                    assert list(got_lists["col_list"][b, h, j, :n].view(np.uint32)) == want, (b, h, j)
                o_ref, lse_ref = A.forward(Qc, Kc, Vc, keep, keep, scale=w.scale)
                check_forward(o_v, lse_v, o_ref, lse_ref, "bf16", f"qk step b{b}h{h}")
                ref = A.backward(Qc, Kc, Vc, Gc, keep, keep, scale=w.scale)
                check_grads([dq_v, dk_v, dv_v], ref, "bf16", f"qk step b{b}h{h}")
            else:
                rows = _rows_sample(rng, len(keep), 48)
                o_ref, lse_ref = A.forward_rows(rows, Qc, Kc, Vc, keep, keep, scale=w.scale)
                check_forward(o_v[rows], lse_v[rows], o_ref, lse_ref, "bf16", f"qk step rows b{b}h{h}")
                dq_ref = A.backward_rows(rows, Qc, Kc, Vc, Gc, keep, keep, scale=w.scale)
                assert rel_fro(dq_v[rows], dq_ref) <= 5e-2, (b, h)
                keys = _rows_sample(rng, len(keep), 24)
                dk_ref, dv_ref = A.backward_key_rows(keys, Qc, Kc, Vc, Gc, keep, keep, scale=w.scale)
                assert rel_fro(dk_v[keys], dk_ref) <= 5e-2, (b, h)
                assert rel_fro(dv_v[keys], dv_ref) <= 5e-2, (b, h)
    note("[workload step] qk ok")


@pytest.mark.timeout(900)
def test_workload5_step_matches_oracle():
    import bench
    import sparse_causal_attention_amd as scfa

    note("[workload step] hash_drop50_fwd_bf16_T1M_nb256: inputs and one step")
    w, step, _, dense_in = bench.workload_setup(scfa, torch, 5)
    assert w.name == "hash_drop50_fwd_bf16_T1M_nb256"
    _, outs = step(None)
    torch.cuda.synchronize()
    q, k, v, _ = dense_in
    rng = np.random.default_rng(1 << 20)
    for h in (0, w.H - 1):
        note(f"[workload step] hash head {h}")
        keep = keep_set(w, 0, h)[0]
        mask = np.zeros(w.T, bool)
        mask[keep] = True
        Rh = lsh_rotation(w, h)
        Q, K, V = (_head(t, 0, h) for t in (q, k, v))
        res = {}
        for which, x, b in (("q", Q, 0), ("k", K, w.B)):  # the sort ran over Q and K stacked along the batch
            p_ref, h_ref, i_ref = lsh.bucket_sort(lsh.buckets_c(x[keep], Rh), keep)
            np.testing.assert_array_equal(to_np(outs["hash"][b, h]), h_ref)
            np.testing.assert_array_equal(to_np(outs["idx"][b, h]), i_ref)
            res[which] = (p_ref, h_ref, i_ref)
        (_, hq, iq), (_, hk, ik) = res["q"], res["k"]
        O, L = _head(outs["o"], 0, h), _head(outs["lse"], 0, h)
        assert np.all(O[~mask] == 0)
        rows = _rows_sample(rng, len(keep), 64)  # rows of the sorted view; view row i is position iq[i]
        o_ref, lse_ref = A.forward_rows(rows, Q[iq], K[ik], V[ik], iq, ik, hq, hk, w.scale)
        check_forward(O[iq[rows]], L[iq[rows]], o_ref, lse_ref, "bf16", f"hash drop step rows h{h}")
    note("[workload step] hash ok")
