"""The benchmark's timed step itself, at full size, against the oracle.

``bench.run_step`` is called exactly as the benchmark times it on the 16k
Hash-sparse training workload (2 x 12 heads, 16,384 tokens, d = 64, 32
buckets): one LSH + sort call over Q and K stacked in one allocation, exact
block lists with tile slots, and the attention kernels reading Q, dO, K and V
through the sort permutations (the ``_lists`` entry points) and writing O, lse
and the gradients at the caller's rows (token order).  Both backward
paths run on the same inputs: the recomputing one the benchmark times by
default, and the stored-dS one (``--stored-ds``).  The oracle recomputes every bucket
id, permutation and block list bit for bit, O, lse and all gradients densely
on two full heads, and sampled query rows and key rows of every other head.
"""

import numpy as np
import pytest

from gen import WORKLOADS, head_inputs, lsh_rotation
from helpers import check_forward, check_grads, note, rel_fro, to_np
from oracle import attention as A
from oracle import blocks as Bk
from oracle import lsh

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _rows_sample(rng, T, n):
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, min(n, T), replace=False)]))


def _check_lists(got, b, h, live, free):
    for i, row in enumerate(Bk.row_lists(live, free)):
        n = int(got["row_count"][b, h, i])
        assert n == len(row), (b, h, i)
        want = [j | (0x80000000 if f else 0) for j, f in row]
        assert list(got["row_list"][b, h, i, :n].view(np.uint32)) == want, (b, h, i)
    for j, colv in enumerate(Bk.col_lists(live, free)):
        n = int(got["col_count"][b, h, j])
        assert n == len(colv), (b, h, j)
        want = [i | (0x80000000 if f else 0) for i, f in colv]
        assert list(got["col_list"][b, h, j, :n].view(np.uint32)) == want, (b, h, j)


@pytest.mark.timeout(600)
def test_timed_step_matches_oracle():
    import bench
    import sparse_causal_attention_amd as scfa

    w = WORKLOADS[bench.WORKLOAD_ID]
    assert w.name == "hash_train_bf16_T16384_nb32"
    note(f"[timed step] {w.name}: inputs")
    q, k, v, do, R, qk = bench.make_inputs(w, torch)
    note("[timed step] run_step (stacked sort, exact lists, permuted rows)")
    meta, outs = bench.run_step(scfa, w, q, k, v, do, R, exact=True, copy_sorted=False, qk=qk)
    note("[timed step] run_step with the stored-dS backward")
    ds = bench.prepare_ds(scfa, torch, w, q, k, R, qk, exact=True)
    meta_ds, outs_ds = bench.run_step(scfa, w, q, k, v, do, R, exact=True, copy_sorted=False, qk=qk, ds=ds)
    torch.cuda.synchronize()
    assert int(meta_ds["col_base"][-1].item()) <= ds.shape[0]  # every tile stored: dQ came from dS
    for cnt, lst in (("row_count", "row_list"), ("col_count", "col_list")):  # entries past a count are unspecified
        assert torch.equal(meta_ds[cnt], meta[cnt])
        valid = torch.arange(meta[lst].shape[-1], device=meta[lst].device) < meta[cnt][..., None]
        assert torch.equal(meta_ds[lst][valid], meta[lst][valid])
    # same forward; dK, dV bit for bit (same kernel, D from the preprocess equals D from the dQ kernel)
    for i in (0, 1, 3, 4):  # O, lse, dK, dV
        assert torch.equal(outs_ds[i], outs[i]), i
    dq_ds = to_np(outs_ds[2])
    got = {n: meta[n].cpu().numpy() for n in ("row_count", "row_list", "col_count", "col_list", "q_hash", "q_idx",
                                              "q_perm", "k_hash", "k_idx", "k_perm")}
    assert meta["outputs"] == "caller rows"
    o, lse, dq, dk, dv = (to_np(t) for t in outs)  # caller (token) order
    del q, k, v, do, qk, meta, outs, ds, meta_ds, outs_ds
    rng = np.random.default_rng(16384)
    full_heads = {(0, 0), (w.B - 1, w.H - 1)}
    for b in range(w.B):
        for h in range(w.H):
            hi = head_inputs(w, b, h)
            Rh = lsh_rotation(w, h)
            # sort results, bit for bit
            res = {}
            for which, x, pos in (("q", hi.q, hi.q_pos), ("k", hi.k, hi.k_pos)):
                p_ref, h_ref, i_ref = lsh.bucket_sort(lsh.buckets_c(x, Rh), pos)
                np.testing.assert_array_equal(got[which + "_perm"][b, h], p_ref)
                np.testing.assert_array_equal(got[which + "_hash"][b, h], h_ref)
                np.testing.assert_array_equal(got[which + "_idx"][b, h], i_ref)
                res[which] = (p_ref, h_ref, i_ref)
            (pq, hq, iq), (pk, hk, ik) = res["q"], res["k"]
            # caller-order outputs seen in the sorted view: view row i is caller row pq[i] (pk for keys)
            o_v, lse_v, dq_v, dqds_v = o[b, h][pq], lse[b, h][pq], dq[b, h][pq], dq_ds[b, h][pq]
            dk_v, dv_v = dk[b, h][pk], dv[b, h][pk]
            # exact block lists, bit for bit
            _, _, live, free = Bk.metadata_exact(iq, ik, hq, hk, w.block)
            _check_lists(got, b, h, live, free)
            # attention outputs (sorted order)
            qs, ks, vs, dos = hi.q[pq], hi.k[pk], hi.v[pk], hi.do[pq]
            if (b, h) in full_heads:
                note(f"[timed step] full oracle b{b}h{h}")
                o_ref, lse_ref = A.forward(qs, ks, vs, iq, ik, hq, hk, w.scale)
                check_forward(o_v, lse_v, o_ref, lse_ref, "bf16", f"step b{b}h{h}")
                ref = A.backward(qs, ks, vs, dos, iq, ik, hq, hk, w.scale)
                check_grads([dq_v, dk_v, dv_v], ref, "bf16", f"step b{b}h{h}")
                check_grads([dqds_v, dk_v, dv_v], ref, "bf16", f"step stored dS b{b}h{h}")
            else:
                rows = _rows_sample(rng, w.Tq, 64)
                o_ref, lse_ref = A.forward_rows(rows, qs, ks, vs, iq, ik, hq, hk, w.scale)
                check_forward(o_v[rows], lse_v[rows], o_ref, lse_ref, "bf16", f"step rows b{b}h{h}")
                dq_ref = A.backward_rows(rows, qs, ks, vs, dos, iq, ik, hq, hk, w.scale)
                assert rel_fro(dq_v[rows], dq_ref) <= 5e-2, (b, h)
                assert rel_fro(dqds_v[rows], dq_ref) <= 5e-2, (b, h)
                keys = _rows_sample(rng, w.Tk, 32)
                dk_ref, dv_ref = A.backward_key_rows(keys, qs, ks, vs, dos, iq, ik, hq, hk, w.scale)
                assert rel_fro(dk_v[keys], dk_ref) <= 5e-2, (b, h)
                assert rel_fro(dv_v[keys], dv_ref) <= 5e-2, (b, h)
            note(f"[timed step] b{b}h{h} ok")
