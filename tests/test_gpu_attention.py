"""GPU parity of the attention forward and backward against the fp64 oracle.

Cases span several tiles with ragged tails, Tq != Tk, unsorted rows, empty
rows (Hash-sparse), empty key sets, d in {64, 128}, block in {64, 128}, bf16
and fp32, and all three modes (dense causal, QK-sparse, Hash-sparse).
"""

import zlib

import numpy as np
import pytest

from gen import bf16_round, synthetic_case
from helpers import check_forward, check_grads, dev, note, to_np
from oracle import attention as A

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _lib():
    import sparse_causal_attention_amd as scfa

    return scfa


def _tdtype(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _positions(c, b, h, Tq, Tk):
    if c.q_idx is None:
        return np.arange(Tq), np.arange(Tk), None, None
    qh = None if c.q_hash is None else c.q_hash[b, h]
    kh = None if c.k_hash is None else c.k_hash[b, h]
    return c.q_idx[b, h], c.k_idx[b, h], qh, kh


def _oracle_fwd(c, scale):
    B, H, Tq, d = c.q.shape
    Tk = c.k.shape[2]
    o = np.zeros((B, H, Tq, d))
    lse = np.zeros((B, H, Tq))
    for b in range(B):
        for h in range(H):
            qi, ki, qh, kh = _positions(c, b, h, Tq, Tk)
            o[b, h], lse[b, h] = A.forward(c.q[b, h], c.k[b, h], c.v[b, h], qi, ki, qh, kh, scale)
    return o, lse


def _oracle_bwd(c, scale):
    B, H, Tq, d = c.q.shape
    Tk = c.k.shape[2]
    out = [np.zeros((B, H, Tq, d)), np.zeros((B, H, Tk, d)), np.zeros((B, H, Tk, d))]
    for b in range(B):
        for h in range(H):
            qi, ki, qh, kh = _positions(c, b, h, Tq, Tk)
            g = A.backward(c.q[b, h], c.k[b, h], c.v[b, h], c.do[b, h], qi, ki, qh, kh, scale)
            for i in range(3):
                out[i][b, h] = g[i]
    return out


def _run(c, mode, block, flags=0, bwd=False):
    scfa = _lib()
    td = _tdtype(c.dtype)
    q, k, v = dev(c.q, td), dev(c.k, td), dev(c.v, td)
    d = c.q.shape[-1]
    scale = 1.0 / np.sqrt(d)
    if mode == "hash":
        idx = [dev(c.q_idx), dev(c.k_idx), dev(c.q_hash), dev(c.k_hash)]
        o, lse = scfa.hash_sparse_fwd(q, k, v, *idx, block=block, scale=scale, flags=flags)
    else:
        idx = [None, None] if mode == "dense" else [dev(c.q_idx), dev(c.k_idx)]
        o, lse = scfa.qk_sparse_fwd(q, k, v, *idx, block=block, scale=scale, flags=flags)
    grads = None
    if bwd:
        do = dev(c.do, td)
        if mode == "hash":
            grads = scfa.hash_sparse_bwd(q, k, v, o, lse, do, *idx, block=block, scale=scale, flags=flags)
        else:
            grads = scfa.qk_sparse_bwd(q, k, v, o, lse, do, *idx, block=block, scale=scale, flags=flags)
    torch.cuda.synchronize()
    return o, lse, grads, scale


# (name, synthetic_case kwargs, mode)
CASES = [
    ("dense_T300", dict(Tq=300, Tk=300, mode="dense"), "dense"),
    ("dense_Tq_lt_Tk", dict(Tq=130, Tk=333, mode="dense"), "dense"),
    ("qk_shared_ascending", dict(Tq=517, Tk=517, mode="qk", shared=True), "qk"),
    ("qk_independent_shuffled", dict(Tq=333, Tk=517, mode="qk", layout="shuffled"), "qk"),
    ("hash_grouped_nb4", dict(Tq=600, Tk=555, mode="hash", nb=4, layout="grouped"), "hash"),
    ("hash_shuffled_nb3", dict(Tq=257, Tk=321, mode="hash", nb=3, layout="shuffled"), "hash"),
    ("hash_shared_grouped_nb8", dict(Tq=700, Tk=700, mode="hash", nb=8, layout="grouped", shared=True), "hash"),
    ("hash_one_bucket", dict(Tq=200, Tk=260, mode="hash", nb=1, layout="grouped"), "hash"),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d,block", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("name,kw,mode", CASES, ids=[c[0] for c in CASES])
def test_forward_backward_parity(name, kw, mode, d, block, dtype):
    seed = zlib.crc32(f"{name}/{d}/{block}/{dtype}".encode()) % 100000
    c = synthetic_case(seed, B=1, H=2, d=d, dtype=dtype, **kw)
    note(f"[fwd+bwd] {name} d={d} block={block} dtype={dtype} Tq={c.q.shape[2]} Tk={c.k.shape[2]}")
    o, lse, grads, scale = _run(c, mode, block, bwd=True)
    o_ref, lse_ref = _oracle_fwd(c, scale)
    check_forward(to_np(o), to_np(lse), o_ref, lse_ref, dtype, name)
    ref = _oracle_bwd(c, scale)
    check_grads([to_np(g) for g in grads], ref, dtype, name)


@pytest.mark.parametrize("mode", ["dense", "qk", "hash"])
def test_pruning_and_mask_flags_are_bit_identical(mode):
    c = synthetic_case(7, B=2, H=2, Tq=450, Tk=450, mode=mode, nb=4, layout="grouped", shared=(mode != "hash"))
    note(f"[flags] {mode}")
    scfa = _lib()
    base = _run(c, mode, 64, bwd=True)
    for flags in (scfa.FLAG_NO_PRUNE, scfa.FLAG_FORCE_MASK, scfa.FLAG_NO_PRUNE | scfa.FLAG_FORCE_MASK):
        other = _run(c, mode, 64, flags=flags, bwd=True)
        assert torch.equal(base[0], other[0]), flags
        assert torch.equal(base[1], other[1]), flags
        for g0, g1 in zip(base[2], other[2]):
            assert torch.equal(g0, g1), flags


def test_repeated_runs_are_bit_identical():
    c = synthetic_case(8, B=1, H=3, Tq=640, Tk=640, mode="hash", nb=4, layout="grouped")
    note("[determinism] hash")
    a = _run(c, "hash", 64, bwd=True)
    b = _run(c, "hash", 64, bwd=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    for x, y in zip(a[2], b[2]):
        assert torch.equal(x, y)


@pytest.mark.parametrize("mode", ["dense", "qk", "hash"])
def test_empty_key_set_gives_zero_rows(mode):
    c = synthetic_case(9, B=1, H=2, Tq=70, Tk=0, mode=mode, nb=2)
    note(f"[Tk=0] {mode}")
    o, lse, grads, _ = _run(c, mode, 64, bwd=True)
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    assert torch.all(grads[0] == 0)


@pytest.mark.parametrize("mode", ["dense", "qk", "hash"])
def test_empty_query_set(mode):
    c = synthetic_case(10, B=1, H=2, Tq=0, Tk=90, mode=mode, nb=2)
    note(f"[Tq=0] {mode}")
    o, lse, grads, _ = _run(c, mode, 64, bwd=True)
    assert o.numel() == 0
    assert torch.all(grads[1] == 0) and torch.all(grads[2] == 0)


def test_single_query_row():
    c = synthetic_case(11, B=1, H=1, Tq=1, Tk=200, mode="qk", T_orig=1000)
    note("[Tq=1]")
    o, lse, grads, scale = _run(c, "qk", 64, bwd=True)
    o_ref, lse_ref = _oracle_fwd(c, scale)
    check_forward(to_np(o), to_np(lse), o_ref, lse_ref, "bf16", "Tq=1")
    check_grads([to_np(g) for g in grads], _oracle_bwd(c, scale), "bf16", "Tq=1")


def test_value_ones_gives_ones():
    """V = 1: every non-empty row of O is exactly 1 (rows of P sum to one)."""
    c = synthetic_case(12, B=1, H=2, Tq=500, Tk=480, mode="hash", nb=4, layout="grouped")
    c.v[:] = 1.0
    note("[V=1]")
    o, lse, _, _ = _run(c, "hash", 64)
    o = to_np(o)
    nonempty = ~np.isneginf(to_np(lse))
    assert np.all(o[nonempty] == 1.0)
    assert np.all(o[~nonempty] == 0.0)


@pytest.mark.parametrize("mode", ["qk", "hash"])
def test_ragged_head_lengths_by_padding(mode):
    """Heads with different kept counts in one padded batch: padding queries at
    position -1, padding keys at 2^31 - 1; every head equals the oracle at its
    own length, and padding rows give 0 (lse -inf) and zero gradients."""
    rng = np.random.default_rng(31 if mode == "qk" else 32)
    B, H, T, d = 2, 3, 640, 64
    nq = rng.integers(60, T + 1, (B, H))
    nk = rng.integers(60, T + 1, (B, H))
    nq[0, 0], nk[0, 1] = T, 1
    Q, K, V, G = (bf16_round(rng.standard_normal((B, H, T, d)).astype(np.float32)) for _ in range(4))
    qi = np.full((B, H, T), -1, np.int32)
    ki = np.full((B, H, T), 2**31 - 1, np.int32)
    qh = rng.integers(0, 5, (B, H, T)).astype(np.int32)
    kh = rng.integers(0, 5, (B, H, T)).astype(np.int32)
    for b in range(B):
        for h in range(H):
            qi[b, h, :nq[b, h]] = np.sort(rng.choice(2 * T, nq[b, h], replace=False))
            ki[b, h, :nk[b, h]] = np.sort(rng.choice(2 * T, nk[b, h], replace=False))
    scfa = _lib()
    note(f"[ragged] {mode}")
    q, k, v, g = (dev(x, torch.bfloat16) for x in (Q, K, V, G))
    idx = (dev(qi), dev(ki))
    if mode == "qk":
        o, lse = scfa.qk_sparse_fwd(q, k, v, *idx)
        grads = scfa.qk_sparse_bwd(q, k, v, o, lse, g, *idx)
    else:
        hs = (dev(qh), dev(kh))
        o, lse = scfa.hash_sparse_fwd(q, k, v, *idx, *hs)
        grads = scfa.hash_sparse_bwd(q, k, v, o, lse, g, *idx, *hs)
    torch.cuda.synchronize()
    o, lse = to_np(o), to_np(lse)
    dq, dk, dv = (to_np(x) for x in grads)
    for b in range(B):
        for h in range(H):
            a, c = nq[b, h], nk[b, h]
            hq = qh[b, h, :a] if mode == "hash" else None
            hk = kh[b, h, :c] if mode == "hash" else None
            o_ref, lse_ref = A.forward(Q[b, h, :a], K[b, h, :c], V[b, h, :c], qi[b, h, :a], ki[b, h, :c], hq, hk)
            check_forward(o[b, h, :a], lse[b, h, :a], o_ref, lse_ref, "bf16", f"ragged {mode} b{b}h{h}")
            ref = A.backward(Q[b, h, :a], K[b, h, :c], V[b, h, :c], G[b, h, :a], qi[b, h, :a], ki[b, h, :c], hq, hk)
            check_grads([dq[b, h, :a], dk[b, h, :c], dv[b, h, :c]], ref, "bf16", f"ragged {mode} b{b}h{h}")
            assert np.all(o[b, h, a:] == 0) and np.all(np.isneginf(lse[b, h, a:]))
            assert np.all(dq[b, h, a:] == 0) and np.all(dk[b, h, c:] == 0) and np.all(dv[b, h, c:] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_exact_lists_are_bit_identical(dtype):
    """Attention over exact lists (fewer tiles) equals attention over range-rule lists bit
    for bit: the extra tiles of the range rule hold no valid pair."""
    scfa = _lib()
    c = synthetic_case(41, B=2, H=3, Tq=1500, Tk=1400, d=64, dtype=dtype, mode="hash", nb=6, layout="grouped")
    note(f"[exact lists] dtype={dtype}")
    td = _tdtype(dtype)
    q, k, v, do = (dev(x).to(td) for x in (c.q, c.k, c.v, c.do))
    qi, ki, qh, kh = (dev(x) for x in (c.q_idx, c.k_idx, c.q_hash, c.k_hash))
    m_range = scfa.block_meta(qi, ki, qh, kh, block=64, with_cols=True)
    m_exact = scfa.block_meta(qi, ki, qh, kh, block=64, with_cols=True, exact=True)
    torch.cuda.synchronize()
    n_range, n_exact = int(m_range["row_count"].sum()), int(m_exact["row_count"].sum())
    assert n_exact < n_range
    assert int(m_exact["col_count"].sum()) == n_exact
    res = []
    for m in (m_range, m_exact):
        o, lse = scfa.attn_fwd_lists(q, k, v, qi, ki, qh, kh, m, block=64)
        dq, delta = scfa.attn_bwd_dq_lists(q, k, v, o, lse, do, qi, ki, qh, kh, m, block=64)
        dk, dv = scfa.attn_bwd_dkdv_lists(q, k, v, lse, do, delta, qi, ki, qh, kh, m, block=64)
        res.append((o, lse, dq, dk, dv))
    torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a, b)


@pytest.mark.parametrize("mode,d,block,Tq,Tk", [("hash", 64, 64, 1500, 1400), ("qk", 64, 64, 777, 1000),
                                                ("dense", 64, 64, 650, 650), ("hash", 128, 128, 1300, 1300),
                                                ("hash", 128, 64, 500, 450), ("hash", 64, 128, 1300, 1250)])
def test_row_indirection_bit_identical(mode, d, block, Tq, Tk):
    """Attention over a permuted view (q_rows / k_rows) equals attention over the gathered copies bit
    for bit, for the forward and both backward kernels; indices out of range behave as clamped."""
    scfa = _lib()
    c = synthetic_case(51, B=2, H=2, Tq=Tq, Tk=Tk, d=d, dtype="bf16", mode="hash" if mode == "hash" else "qk",
                       nb=5, layout="grouped")
    note(f"[row indirection] {mode} d={d} block={block} Tq={Tq} Tk={Tk}")
    q, k, v, do = (dev(x).to(torch.bfloat16) for x in (c.q, c.k, c.v, c.do))
    if mode == "dense":
        qi = ki = qh = kh = None
    else:
        qi, ki = dev(c.q_idx), dev(c.k_idx)
        qh, kh = (dev(c.q_hash), dev(c.k_hash)) if mode == "hash" else (None, None)
    g = torch.Generator(device="cuda:0")
    g.manual_seed(9)
    qr = torch.stack([torch.stack([torch.randperm(Tq, generator=g, device="cuda:0") for _ in range(2)])
                      for _ in range(2)]).to(torch.int32)
    kr = torch.stack([torch.stack([torch.randperm(Tk, generator=g, device="cuda:0") for _ in range(2)])
                      for _ in range(2)]).to(torch.int32)
    qr[0, 0, 3], kr[1, 1, 5] = -7, Tk + 11  # out of range: clamped on the device
    gather = lambda x, r, T: torch.gather(  # noqa: E731
        x, 2, r.clamp(0, T - 1).long()[..., None].expand(-1, -1, -1, x.shape[-1]).contiguous())
    qs, dos = gather(q, qr, Tq), gather(do, qr, Tq)
    ks, vs = gather(k, kr, Tk), gather(v, kr, Tk)
    meta = None if mode == "dense" else scfa.block_meta(qi, ki, qh, kh, block=block, with_cols=True, exact=True)
    o1, l1 = scfa.attn_fwd_lists(qs, ks, vs, qi, ki, qh, kh, meta, block=block)
    dq1, de1 = scfa.attn_bwd_dq_lists(qs, ks, vs, o1, l1, dos, qi, ki, qh, kh, meta, block=block)
    dk1, dv1 = scfa.attn_bwd_dkdv_lists(qs, ks, vs, l1, dos, de1, qi, ki, qh, kh, meta, block=block)
    o2, l2 = scfa.attn_fwd_lists(q, k, v, qi, ki, qh, kh, meta, block=block, q_rows=qr, k_rows=kr)
    dq2, de2 = scfa.attn_bwd_dq_lists(q, k, v, o2, l2, do, qi, ki, qh, kh, meta, block=block, q_rows=qr, k_rows=kr)
    dk2, dv2 = scfa.attn_bwd_dkdv_lists(q, k, v, l2, do, de2, qi, ki, qh, kh, meta, block=block, q_rows=qr,
                                        k_rows=kr)
    torch.cuda.synchronize()
    for a_, b_ in [(o1, o2), (l1, l2), (dq1, dq2), (de1, de2), (dk1, dk2), (dv1, dv2)]:
        assert torch.equal(a_, b_)


@pytest.mark.parametrize("mode,Tq,Tk", [("hash", 1500, 1400), ("qk", 777, 1000), ("dense", 650, 650)])
def test_d128_block128_lists_equal_block64_lists(mode, Tq, Tk):
    """At d = 128, block-128 lists run as one 128-query group per block (dense, QK-sparse) or as two
    64-query groups walking the same list (Hash-sparse).  Either way a query sees the chunks of its
    block-64 list plus chunks whose keys are all masked for it (exact zero terms, no change of the
    running max), in the same order and key halves, and some free tiles masked, so the result equals
    the block-64 lists' bit for bit."""
    scfa = _lib()
    c = synthetic_case(52, B=2, H=2, Tq=Tq, Tk=Tk, d=128, dtype="bf16", mode="hash" if mode == "hash" else "qk",
                       nb=5, layout="grouped")
    note(f"[block-128 lists in 64-query groups] {mode} Tq={Tq} Tk={Tk}")
    q, k, v = (dev(x).to(torch.bfloat16) for x in (c.q, c.k, c.v))
    if mode == "dense":
        qi = ki = qh = kh = None
    else:
        qi, ki = dev(c.q_idx), dev(c.k_idx)
        qh, kh = (dev(c.q_hash), dev(c.k_hash)) if mode == "hash" else (None, None)
    res = []
    for block in (64, 128):
        meta = None if mode == "dense" else scfa.block_meta(qi, ki, qh, kh, block=block, with_cols=False, exact=True)
        res.append(scfa.attn_fwd_lists(q, k, v, qi, ki, qh, kh, meta, block=block))
    if mode == "hash":
        res.append(scfa.hash_sparse_fwd(q, k, v, qi, ki, qh, kh, block=128))
    torch.cuda.synchronize()
    for o_, l_ in res[1:]:
        assert torch.equal(o_, res[0][0]) and torch.equal(l_, res[0][1])


@pytest.mark.parametrize("d,block", [(64, 64), (128, 128)])
def test_key_half_merge_with_one_empty_half_and_wide_scores(d, block):
    """The forward splits every 64-key chunk into two halves handled by different waves and merges
    their softmax states at the end.  Keys 0-31 of every chunk are in bucket 0 and keys 32-63 in
    bucket 1, so each query's admissible keys all lie in its bucket's half of each chunk and the
    other half's state stays empty (reference max -inf); random query positions also leave some
    rows with no admissible key at all and cut others inside a chunk.  Scores are widened (inputs
    scaled by 4, score std about 16) so the lazy rescale fires often and the merge's factors span a
    wide range."""
    rng = np.random.default_rng(71 + d)
    B, H, Tq, Tk = 1, 2, 320, 448
    q = bf16_round(4.0 * rng.standard_normal((B, H, Tq, d), dtype=np.float32))
    k = bf16_round(4.0 * rng.standard_normal((B, H, Tk, d), dtype=np.float32))
    v = bf16_round(rng.standard_normal((B, H, Tk, d), dtype=np.float32))
    k_hash = np.broadcast_to(((np.arange(Tk) % 64) >= 32).astype(np.int32), (B, H, Tk)).copy()
    k_idx = np.broadcast_to(np.arange(Tk, dtype=np.int32) * 2, (B, H, Tk)).copy()
    q_hash = np.broadcast_to((np.arange(Tq) % 2).astype(np.int32), (B, H, Tq)).copy()
    q_idx = np.broadcast_to(rng.integers(0, 2 * Tk + 8, size=Tq).astype(np.int32), (B, H, Tq)).copy()
    note(f"[key-half merge] d={d} block={block}")
    scfa = _lib()
    tq, tk, tv = (dev(x, torch.bfloat16) for x in (q, k, v))
    o, lse = scfa.hash_sparse_fwd(tq, tk, tv, dev(q_idx), dev(k_idx), dev(q_hash), dev(k_hash), block=block)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(d)
    for h in range(H):
        o_ref, lse_ref = A.forward(q[0, h], k[0, h], v[0, h], q_idx[0, h], k_idx[0, h], q_hash[0, h], k_hash[0, h],
                                   scale)
        check_forward(to_np(o[0, h]), to_np(lse[0, h]), o_ref, lse_ref, "bf16", f"key-half merge h={h}")
