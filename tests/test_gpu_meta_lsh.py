"""Bit-exact GPU parity of block metadata, LSH bucket ids and the bucket sort."""

import json
import os

import numpy as np
import pytest

from gen import bf16_round, synthetic_case
from helpers import dev, note
from oracle import blocks as Bk
from oracle import lsh

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _scfa():
    import sparse_causal_attention_amd as scfa

    return scfa


def _compare_meta(out, c, block, exact=False, heads=None):
    B, H, Tq = c.q_idx.shape
    hashed = c.q_hash is not None
    got = {k: v.cpu().numpy() for k, v in out.items() if hasattr(v, "cpu")}
    for b in range(B):
        for h in range(H):
            if heads is not None and (b, h) not in heads:
                continue
            qh = c.q_hash[b, h] if hashed else None
            kh = c.k_hash[b, h] if hashed else None
            if exact:
                qs, ks, live, free = Bk.metadata_exact(c.q_idx[b, h], c.k_idx[b, h], qh, kh, block)
            else:
                qs, ks, live, free = Bk.metadata(c.q_idx[b, h], c.k_idx[b, h], qh, kh, block)
            np.testing.assert_array_equal(got["q_stats"][b, h], qs)
            np.testing.assert_array_equal(got["k_stats"][b, h], ks)
            for i, row in enumerate(Bk.row_lists(live, free)):
                n = got["row_count"][b, h, i]
                assert n == len(row), (b, h, i)
                want = [j | (0x80000000 if f else 0) for j, f in row]
                assert list(got["row_list"][b, h, i, :n].view(np.uint32)) == want
            for j, colv in enumerate(Bk.col_lists(live, free)):
                n = got["col_count"][b, h, j]
                assert n == len(colv), (b, h, j)
                want = [i | (0x80000000 if f else 0) for i, f in colv]
                assert list(got["col_list"][b, h, j, :n].view(np.uint32)) == want


@pytest.mark.parametrize("block", [64, 128])
@pytest.mark.parametrize(
    "kw",
    [
        dict(Tq=700, Tk=700, mode="qk", shared=True),
        dict(Tq=333, Tk=1111, mode="qk", layout="shuffled"),
        dict(Tq=1000, Tk=900, mode="hash", nb=6, layout="grouped"),
        dict(Tq=513, Tk=257, mode="hash", nb=3, layout="shuffled"),
        dict(Tq=5000, Tk=5000, mode="hash", nb=16, layout="grouped", shared=True),
    ],
)
def test_block_meta_bit_exact(kw, block):
    c = synthetic_case(21, B=2, H=2, **kw)
    note(f"[meta] {kw} block={block}")
    out = _scfa().block_meta(dev(c.q_idx), dev(c.k_idx),
                             None if c.q_hash is None else dev(c.q_hash),
                             None if c.k_hash is None else dev(c.k_hash), block=block)
    torch.cuda.synchronize()
    _compare_meta(out, c, block)


@pytest.mark.parametrize("block", [64, 128])
@pytest.mark.parametrize(
    "kw",
    [
        dict(Tq=700, Tk=700, mode="qk", shared=True),
        dict(Tq=1000, Tk=900, mode="hash", nb=6, layout="grouped"),
        dict(Tq=513, Tk=257, mode="hash", nb=3, layout="shuffled"),
        dict(Tq=5000, Tk=5000, mode="hash", nb=16, layout="grouped", shared=True),
        dict(Tq=3000, Tk=2500, mode="hash", nb=150, layout="grouped"),  # many blocks with > 3 buckets
        dict(Tq=1, Tk=130, mode="hash", nb=2, layout="grouped"),
        dict(Tq=777, Tk=901, mode="hash", nb=40, layout="shuffled"),  # up to a bucket per row, unsorted
        dict(Tq=1200, Tk=1200, mode="hash", nb=1000, layout="grouped", shared=True),
    ],
)
def test_block_meta_exact_bit_exact(kw, block):
    c = synthetic_case(22, B=2, H=2, **kw)
    note(f"[meta exact] {kw} block={block}")
    out = _scfa().block_meta(dev(c.q_idx), dev(c.k_idx),
                             None if c.q_hash is None else dev(c.q_hash),
                             None if c.k_hash is None else dev(c.k_hash), block=block, exact=True)
    torch.cuda.synchronize()
    _compare_meta(out, c, block, exact=True)


def _lsh_case(seed, B, H, T, d, nb, dtype="bf16"):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, H, T, d), dtype=np.float32)
    if dtype == "bf16":
        x = bf16_round(x)
    R = rng.standard_normal((H, d, nb // 2), dtype=np.float32)
    return x, R


@pytest.mark.parametrize(
    "B,H,T,d,nb,dtype",
    [(1, 2, 1000, 64, 16, "bf16"), (2, 3, 4099, 64, 32, "bf16"), (1, 2, 9000, 128, 256, "bf16"),
     (1, 1, 777, 64, 2, "fp32"), (1, 2, 3000, 128, 1024, "bf16"), (1, 1, 1, 64, 4, "bf16"),
     (1, 1, 40000, 64, 256, "bf16"), (2, 1, 33000, 64, 512, "fp32")],  # the last two: two-level scan
)
def test_lsh_sort_bit_exact(B, H, T, d, nb, dtype):
    x, R = _lsh_case(B * 1000 + T, B, H, T, d, nb, dtype)
    note(f"[lsh] B={B} H={H} T={T} d={d} nb={nb} {dtype}")
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    xt = dev(x, td)
    comp = dev(x[..., ::-1].copy(), td)  # any second tensor
    hs, ids, perm, xs, cs = _scfa().lsh_bucket_sort(xt, dev(R), nb, companion=comp)
    torch.cuda.synchronize()
    hs, ids, perm = hs.cpu().numpy(), ids.cpu().numpy(), perm.cpu().numpy()
    for b in range(B):
        for h in range(H):
            bk = lsh.buckets_c(x[b, h], R[h])
            p_ref, h_ref, i_ref = lsh.bucket_sort(bk, np.arange(T))
            np.testing.assert_array_equal(perm[b, h], p_ref)
            np.testing.assert_array_equal(hs[b, h], h_ref)
            np.testing.assert_array_equal(ids[b, h], i_ref)
    assert torch.equal(xs, xt[torch.arange(B)[:, None, None], torch.arange(H)[None, :, None],
                              torch.from_numpy(perm).long().cuda()])
    assert torch.equal(cs, comp[torch.arange(B)[:, None, None], torch.arange(H)[None, :, None],
                                torch.from_numpy(perm).long().cuda()])


@pytest.mark.parametrize("d,nb,T", [(64, 16, 5000), (128, 256, 3000), (128, 8, 2000), (64, 64, 4097)])
def test_lsh_near_ties_bit_exact(d, nb, T):
    """R with exactly duplicated columns, columns one float32 ulp apart and a negated column:
    many tokens' two best candidates tie or nearly tie, so the bf16 matrix-core projection
    cannot decide them and the float64 recomputation must (first maximum, sequential sums)."""
    H = 2
    x, R = _lsh_case(77 + d + nb, 1, H, T, d, nb)
    half = nb // 2
    for c in range(1, half, 4):
        R[:, :, c] = R[:, :, c - 1]  # exact ties
    for c in range(2, half, 4):
        R[:, :, c] = np.nextafter(R[:, :, c - 2], np.float32(np.inf))  # one ulp apart
    if half >= 4:
        R[:, :, 3] = -R[:, :, 0]  # p_3 = -p_0: ties between +p and -p candidates
    x[0, :, ::97] = 0.0  # all-zero rows: every candidate ties at 0, the first (bucket 0) wins
    note(f"[lsh near ties] d={d} nb={nb} T={T}")
    hs, ids, perm, _, _ = _scfa().lsh_bucket_sort(dev(x, torch.bfloat16), dev(R), nb, want_x=False)
    torch.cuda.synchronize()
    for h in range(H):
        bk = lsh.buckets_c(x[0, h], R[h])
        p_ref, h_ref, i_ref = lsh.bucket_sort(bk, np.arange(T))
        np.testing.assert_array_equal(perm[0, h].cpu().numpy(), p_ref)
        np.testing.assert_array_equal(hs[0, h].cpu().numpy(), h_ref)
        assert (bk[::97] == 0).all()


@pytest.mark.parametrize("ascending_flag,T", [(False, 6000), (True, 6000), (False, 40000)])
def test_lsh_sort_with_given_positions(ascending_flag, T):
    """Explicit positions: shuffled (five-pass sort) and ascending (one pass with the flag);
    at 40000 tokens the position passes use the two-level scan."""
    B, H, d, nb = 1, 2, 64, 8
    x, R = _lsh_case(5, B, H, T, d, nb)
    rng = np.random.default_rng(6)
    pos = np.stack([np.sort(rng.choice(3 * T, T, replace=False)) for _ in range(H)]).astype(np.int32)[None]
    if not ascending_flag:
        sh = rng.permutation(T)
        pos = pos[..., sh]
        x = x[:, :, sh]
    note(f"[lsh idx] ascending={ascending_flag} T={T}")
    hs, ids, perm, xs, _ = _scfa().lsh_bucket_sort(dev(x, torch.bfloat16), dev(R), nb, idx=dev(pos),
                                                    idx_ascending=ascending_flag)
    torch.cuda.synchronize()
    for h in range(H):
        bk = lsh.buckets_c(x[0, h], R[h])
        p_ref, h_ref, i_ref = lsh.bucket_sort(bk, pos[0, h])
        np.testing.assert_array_equal(perm[0, h].cpu().numpy(), p_ref)
        np.testing.assert_array_equal(hs[0, h].cpu().numpy(), h_ref)
        np.testing.assert_array_equal(ids[0, h].cpu().numpy(), i_ref)


def test_lsh_golden_accumulation_order_and_ties():
    g = json.load(open(os.path.join(GOLDEN, "lsh_sequential_order.json")))
    t = json.load(open(os.path.join(GOLDEN, "lsh_first_max_ties.json")))
    d = g["d"]
    x = np.zeros((1, 1, 1 + len(t["cases"]), d), dtype=np.float32)
    R = np.zeros((1, d, 2), dtype=np.float32)
    for k, val in g["x_nonzero"].items():
        x[0, 0, 0, int(k)] = val
    # the tie cases use R = identity on coordinates 0, 1; place them on
    # coordinates 4, 5 with the same R columns extended there
    for k, c, val in g["R_nonzero"]:
        R[0, k, c] = val
    R[0, 4, 0] = R[0, 5, 1] = 1.0
    for i, case in enumerate(t["cases"]):
        x[0, 0, 1 + i, 4:6] = case["x01"]
    want = [g["expected_bucket"]] + [c["bucket"] for c in t["cases"]]
    note("[lsh golden]")
    hs, ids, perm, _, _ = _scfa().lsh_bucket_sort(dev(x, torch.bfloat16), dev(R), 4, want_x=False)
    torch.cuda.synchronize()
    got = np.empty(x.shape[2], dtype=np.int64)
    got[perm[0, 0].cpu().numpy()] = hs[0, 0].cpu().numpy()
    assert got.tolist() == want


def test_lsh_sort_of_stacked_q_and_k():
    """Q and K in one [2B, H, T, d] allocation (Q first), as the benchmark step passes them: one
    call orders both, and each half matches the oracle for its own tensor with the shared R."""
    B, H, T, d, nb = 2, 3, 3000, 64, 32
    xq, R = _lsh_case(91, B, H, T, d, nb)
    xk, _ = _lsh_case(92, B, H, T, d, nb)
    x = np.concatenate([xq, xk])
    note(f"[lsh stacked q,k] B={B} H={H} T={T}")
    hs, ids, perm, _, _ = _scfa().lsh_bucket_sort(dev(x, torch.bfloat16), dev(R), nb, want_x=False)
    torch.cuda.synchronize()
    hs, ids, perm = hs.cpu().numpy(), ids.cpu().numpy(), perm.cpu().numpy()
    for half, src in enumerate((xq, xk)):
        for b in range(B):
            for h in range(H):
                bk = lsh.buckets_c(src[b, h], R[h])
                p_ref, h_ref, i_ref = lsh.bucket_sort(bk, np.arange(T))
                np.testing.assert_array_equal(perm[half * B + b, h], p_ref)
                np.testing.assert_array_equal(hs[half * B + b, h], h_ref)
                np.testing.assert_array_equal(ids[half * B + b, h], i_ref)
