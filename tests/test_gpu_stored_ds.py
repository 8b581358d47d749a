"""The stored-dS backward: tile slots, gradients, and the fallback.

The dK/dV kernel stores every live tile's bf16 dS^T in a slot of the tile
numbering (scfa_tile_slots) and dQ becomes a block-sparse product over those
tiles.  The slot numbering is index work, compared bit for bit with its
definition; gradients are compared with the fp64 oracle, and dK, dV and D bit
for bit with the recomputing path (same kernels and sums, only the extra
stores differ).  A buffer one tile too small must fall back to the
recomputing dQ kernel, bit-identical to it.
"""

import numpy as np
import pytest

from gen import synthetic_case
from helpers import check_grads, dev, note, rel_fro, to_np
from oracle import attention as A

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _lib():
    import sparse_causal_attention_amd as scfa

    return scfa


@pytest.mark.parametrize("kw,block", [
    (dict(Tq=1500, Tk=1400, mode="hash", nb=6, layout="grouped"), 64),
    (dict(Tq=777, Tk=1000, mode="qk"), 64),
    (dict(Tq=900, Tk=1300, mode="hash", nb=4, layout="shuffled"), 128),
    (dict(Tq=64, Tk=1, mode="hash", nb=2, layout="grouped"), 64),
])
def test_tile_slots_definition(kw, block):
    scfa = _lib()
    c = synthetic_case(61, B=2, H=3, **kw)
    note(f"[tile slots] {kw} block={block}")
    qi, ki = dev(c.q_idx), dev(c.k_idx)
    qh, kh = (dev(c.q_hash), dev(c.k_hash)) if c.q_hash is not None else (None, None)
    meta = scfa.tile_slots(scfa.block_meta(qi, ki, qh, kh, block=block, with_cols=True, exact=True))
    torch.cuda.synchronize()
    rc, rl = meta["row_count"].cpu().numpy(), meta["row_list"].cpu().numpy() & 0x7FFFFFFF
    cc, cl = meta["col_count"].cpu().numpy(), meta["col_list"].cpu().numpy() & 0x7FFFFFFF
    base, rs = meta["col_base"].cpu().numpy(), meta["row_slot"].cpu().numpy()
    B, H, nq, nk = rl.shape
    flat = cc.reshape(-1).astype(np.int64)
    np.testing.assert_array_equal(base, np.concatenate([[0], np.cumsum(flat)]))
    for b in range(B):
        for h in range(H):
            for i in range(nq):
                for t in range(rc[b, h, i]):
                    j = rl[b, h, i, t]
                    rank = list(cl[b, h, j, : cc[b, h, j]]).index(i)
                    assert rs[b, h, i, t] == base[(b * H + h) * nk + j] + rank, (b, h, i, t)


def _run(scfa, q, k, v, do, qi, ki, qh, kh, meta, block, rows, ds):
    o, lse = scfa.attn_fwd_lists(q, k, v, qi, ki, qh, kh, meta, block=block, **rows)
    dq0, delta0 = scfa.attn_bwd_dq_lists(q, k, v, o, lse, do, qi, ki, qh, kh, meta, block=block, **rows)
    dk0, dv0 = scfa.attn_bwd_dkdv_lists(q, k, v, lse, do, delta0, qi, ki, qh, kh, meta, block=block, **rows)
    delta = scfa.attn_bwd_prep(o, lse, do, q_rows=rows.get("q_rows"))
    dk, dv = scfa.attn_bwd_dkdv_ds_lists(q, k, v, lse, do, delta, qi, ki, qh, kh, meta, ds, block=block, **rows)
    dq = scfa.attn_bwd_dq_ds_lists(q, k, v, o, lse, do, qi, ki, qh, kh, meta, ds, delta, block=block, **rows)
    return (dq0, dk0, dv0, delta0), (dq, dk, dv, delta)


@pytest.mark.parametrize("mode,d,block,Tq,Tk,rows", [
    ("hash", 64, 64, 1500, 1400, False), ("hash", 64, 64, 1500, 1400, True), ("qk", 64, 64, 777, 1000, True),
    ("hash", 128, 128, 1300, 1300, True), ("hash", 128, 64, 500, 450, False), ("hash", 64, 128, 1000, 999, True),
    ("qk", 128, 64, 333, 700, False)])
def test_stored_ds_backward(mode, d, block, Tq, Tk, rows):
    scfa = _lib()
    B, H = 2, 2
    c = synthetic_case(62, B=B, H=H, Tq=Tq, Tk=Tk, d=d, dtype="bf16", mode=mode, nb=5, layout="grouped")
    note(f"[stored dS] {mode} d={d} block={block} Tq={Tq} Tk={Tk} rows={rows}")
    q, k, v, do = (dev(x).to(torch.bfloat16) for x in (c.q, c.k, c.v, c.do))
    qi, ki = dev(c.q_idx), dev(c.k_idx)
    qh, kh = (dev(c.q_hash), dev(c.k_hash)) if mode == "hash" else (None, None)
    r = {}
    perm_q = perm_k = None
    if rows:
        g = torch.Generator(device="cuda:0")
        g.manual_seed(5)
        perm_q = torch.stack([torch.stack([torch.randperm(Tq, generator=g, device="cuda:0") for _ in range(H)])
                              for _ in range(B)]).to(torch.int32)
        perm_k = torch.stack([torch.stack([torch.randperm(Tk, generator=g, device="cuda:0") for _ in range(H)])
                              for _ in range(B)]).to(torch.int32)
        r = {"q_rows": perm_q, "k_rows": perm_k}
    meta = scfa.tile_slots(scfa.block_meta(qi, ki, qh, kh, block=block, with_cols=True, exact=True))
    torch.cuda.synchronize()
    total = int(meta["col_base"][-1].item())
    ds = scfa.ds_buffer(total, block)
    ref, got = _run(scfa, q, k, v, do, qi, ki, qh, kh, meta, block, r, ds)
    torch.cuda.synchronize()
    # same kernels and sums as the recomputing path: D, dK, dV bit for bit
    assert torch.equal(got[3], ref[3]), "delta differs"
    assert torch.equal(got[1], ref[1]) and torch.equal(got[2], ref[2]), "dK/dV differ"
    assert rel_fro(to_np(got[0]), to_np(ref[0])) <= 1e-2
    # against the oracle (view order: the rows the kernels read)
    pq = perm_q.cpu().numpy() if rows else None
    pk = perm_k.cpu().numpy() if rows else None
    for b in range(B):
        for h in range(H):
            Qv = c.q[b, h][pq[b, h]] if rows else c.q[b, h]
            dOv = c.do[b, h][pq[b, h]] if rows else c.do[b, h]
            Kv = c.k[b, h][pk[b, h]] if rows else c.k[b, h]
            Vv = c.v[b, h][pk[b, h]] if rows else c.v[b, h]
            gref = A.backward(Qv, Kv, Vv, dOv, c.q_idx[b, h], c.k_idx[b, h],
                              None if mode != "hash" else c.q_hash[b, h], None if mode != "hash" else c.k_hash[b, h],
                              1.0 / np.sqrt(d))
            check_grads([to_np(got[0])[b, h], to_np(got[1])[b, h], to_np(got[2])[b, h]], gref, "bf16",
                        f"stored dS b{b}h{h}")


def test_stored_ds_falls_back_when_the_buffer_is_small():
    scfa = _lib()
    c = synthetic_case(63, B=1, H=3, Tq=1200, Tk=1100, d=64, dtype="bf16", mode="hash", nb=4, layout="grouped")
    note("[stored dS fallback]")
    q, k, v, do = (dev(x).to(torch.bfloat16) for x in (c.q, c.k, c.v, c.do))
    qi, ki, qh, kh = (dev(x) for x in (c.q_idx, c.k_idx, c.q_hash, c.k_hash))
    meta = scfa.tile_slots(scfa.block_meta(qi, ki, qh, kh, block=64, with_cols=True, exact=True))
    torch.cuda.synchronize()
    total = int(meta["col_base"][-1].item())
    assert total > 1
    for cap in (total - 1, 0):
        ds = scfa.ds_buffer(cap, 64)
        ref, got = _run(scfa, q, k, v, do, qi, ki, qh, kh, meta, 64, {}, ds)
        torch.cuda.synchronize()
        for a_, b_ in zip(ref, got):
            assert torch.equal(a_, b_), f"capacity {cap}"


@pytest.mark.parametrize("mode,d,block,Tq,Tk", [("hash", 64, 64, 1500, 1400), ("qk", 64, 64, 777, 1000),
                                                ("hash", 128, 128, 900, 1100), ("hash", 64, 128, 500, 450)])
def test_outputs_at_caller_rows(mode, d, block, Tq, Tk):
    """SCFA_FLAG_ORIG_ROWS: the forward, both backward paths and the preprocess read and write at the
    caller's rows; every result equals the view-ordered one put back with scatter_rows, bit for bit."""
    scfa = _lib()
    B, H = 2, 2
    c = synthetic_case(64, B=B, H=H, Tq=Tq, Tk=Tk, d=d, dtype="bf16", mode=mode, nb=5, layout="grouped")
    note(f"[caller rows] {mode} d={d} block={block} Tq={Tq} Tk={Tk}")
    q, k, v, do = (dev(x).to(torch.bfloat16) for x in (c.q, c.k, c.v, c.do))
    qi, ki = dev(c.q_idx), dev(c.k_idx)
    qh, kh = (dev(c.q_hash), dev(c.k_hash)) if mode == "hash" else (None, None)
    g = torch.Generator(device="cuda:0")
    g.manual_seed(11)
    qr = torch.stack([torch.stack([torch.randperm(Tq, generator=g, device="cuda:0") for _ in range(H)])
                      for _ in range(B)]).to(torch.int32)
    kr = torch.stack([torch.stack([torch.randperm(Tk, generator=g, device="cuda:0") for _ in range(H)])
                      for _ in range(B)]).to(torch.int32)
    rows = {"q_rows": qr, "k_rows": kr}
    F = scfa.FLAG_ORIG_ROWS
    meta = scfa.tile_slots(scfa.block_meta(qi, ki, qh, kh, block=block, with_cols=True, exact=True))
    torch.cuda.synchronize()
    ds = scfa.ds_buffer(int(meta["col_base"][-1].item()), block)
    # view order
    o, lse = scfa.attn_fwd_lists(q, k, v, qi, ki, qh, kh, meta, block=block, **rows)
    dq, delta = scfa.attn_bwd_dq_lists(q, k, v, o, lse, do, qi, ki, qh, kh, meta, block=block, **rows)
    dk, dv = scfa.attn_bwd_dkdv_lists(q, k, v, lse, do, delta, qi, ki, qh, kh, meta, block=block, **rows)
    # caller order
    o2, lse2 = scfa.attn_fwd_lists(q, k, v, qi, ki, qh, kh, meta, block=block, flags=F, **rows)
    dq2, delta2 = scfa.attn_bwd_dq_lists(q, k, v, o2, lse2, do, qi, ki, qh, kh, meta, block=block, flags=F, **rows)
    dk2, dv2 = scfa.attn_bwd_dkdv_lists(q, k, v, lse2, do, delta2, qi, ki, qh, kh, meta, block=block, flags=F,
                                        **rows)
    delta3 = scfa.attn_bwd_prep(o2, lse2, do, q_rows=qr, flags=F)
    dk3, dv3 = scfa.attn_bwd_dkdv_ds_lists(q, k, v, lse2, do, delta3, qi, ki, qh, kh, meta, ds, block=block, flags=F,
                                           **rows)
    dq3 = scfa.attn_bwd_dq_ds_lists(q, k, v, o2, lse2, do, qi, ki, qh, kh, meta, ds, delta3, block=block, flags=F,
                                    **rows)
    dq_v = scfa.attn_bwd_dq_ds_lists(q, k, v, o, lse, do, qi, ki, qh, kh, meta, ds, delta, block=block, **rows)
    torch.cuda.synchronize()
    un = lambda x, r, T: scfa.scatter_rows(x, r, T, zero_fill=False)  # noqa: E731
    assert torch.equal(o2, un(o, qr, Tq))
    lse_back = torch.empty_like(lse)
    lse_back.scatter_(2, qr.long(), lse)
    assert torch.equal(lse2, lse_back)
    assert torch.equal(delta2, delta) and torch.equal(delta3, delta)  # delta stays in view order
    assert torch.equal(dq2, un(dq, qr, Tq))
    assert torch.equal(dk2, un(dk, kr, Tk)) and torch.equal(dv2, un(dv, kr, Tk))
    assert torch.equal(dk3, dk2) and torch.equal(dv3, dv2)
    assert torch.equal(dq3, un(dq_v, qr, Tq))
