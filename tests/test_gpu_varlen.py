"""Packed ragged heads: every head with its own query and key counts, back to back.

Dropping tokens per head gives each head its own kept count (SCFA page, "SCFA
solution > 1. QK-Sparse": compact tensors).  The varlen entry points take the
heads packed with no padding, through per-head offsets.  Every head is compared
with the fp64 oracle at its own length (forward and gradients), including heads
with no queries or no keys; the padded layout (sentinel positions) must give
the same rows bit for bit.
"""

import numpy as np
import pytest

from gen import bf16_round
from helpers import check_forward, check_grads, dev, note, to_np
from oracle import attention as A

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _lib():
    import sparse_causal_attention_amd as scfa

    return scfa


def _heads(seed, lq, lk, d, mode, nb, dtype):
    rng = np.random.default_rng(seed)
    out = []
    for tq, tk in zip(lq, lk):
        T0 = 2 * max(tq, tk, 1)
        qi = np.sort(rng.choice(T0, tq, replace=False)).astype(np.int32)
        ki = np.sort(rng.choice(T0, tk, replace=False)).astype(np.int32)
        qh = rng.integers(0, nb, tq).astype(np.int32) if mode == "hash" else None
        kh = rng.integers(0, nb, tk).astype(np.int32) if mode == "hash" else None
        if mode == "hash":  # rows in (bucket, position) order, as after the sort
            oq, ok = np.lexsort((qi, qh)), np.lexsort((ki, kh))
            qi, qh, ki, kh = qi[oq], qh[oq], ki[ok], kh[ok]
        if mode == "dense":
            qi, ki = np.arange(tq, dtype=np.int32), np.arange(tk, dtype=np.int32)
        arr = [rng.standard_normal((n, d), dtype=np.float32) for n in (tq, tk, tk, tq)]
        if dtype == "bf16":
            arr = [bf16_round(a) for a in arr]
        out.append(dict(q=arr[0], k=arr[1], v=arr[2], do=arr[3], qi=qi, ki=ki, qh=qh, kh=kh))
    return out


def _offsets(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


@pytest.mark.parametrize("mode,d,block,dtype", [("qk", 64, 64, "bf16"), ("hash", 64, 64, "bf16"),
                                                ("hash", 128, 128, "bf16"), ("dense", 64, 64, "bf16"),
                                                ("qk", 64, 64, "fp32"), ("hash", 128, 64, "fp32")])
def test_varlen_matches_oracle_per_head(mode, d, block, dtype):
    scfa = _lib()
    B, H = 2, 3
    if mode == "dense":
        lq = lk = [700, 0, 1300, 64, 1, 999]
    else:
        lq, lk = [700, 0, 1300, 64, 1, 999], [650, 300, 1300, 65, 0, 1000]
    heads = _heads(80 + d + block, lq, lk, d, mode, 5, dtype)
    note(f"[varlen] {mode} d={d} block={block} {dtype} lq={lq} lk={lk}")
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    cat = lambda key, dt=None: dev(np.concatenate([h[key] for h in heads]), dt)  # noqa: E731
    q, k, v, do = cat("q", td), cat("k", td), cat("v", td), cat("do", td)
    qo, ko = dev(_offsets(lq)), dev(_offsets(lk))
    qi = ki = qh = kh = None
    if mode != "dense":
        qi, ki = cat("qi"), cat("ki")
    if mode == "hash":
        qh, kh = cat("qh"), cat("kh")
    mt = dict(H=H, max_Tq=max(lq), max_Tk=max(lk))
    meta = None
    if mode != "dense":
        meta = scfa.block_meta_varlen(qo, ko, qi, ki, qh, kh, block=block, **mt)
    o, lse = scfa.attn_fwd_varlen(q, k, v, qo, ko, qi, ki, qh, kh, meta, block=block, **mt)
    dq, delta = scfa.attn_bwd_dq_varlen(q, k, v, o, lse, do, qo, ko, qi, ki, qh, kh, meta, block=block, **mt)
    dk, dv = scfa.attn_bwd_dkdv_varlen(q, k, v, lse, do, delta, qo, ko, qi, ki, qh, kh, meta, block=block, **mt)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (to_np(t) for t in (o, lse, dq, dk, dv))
    oq, ok = _offsets(lq), _offsets(lk)
    scale = 1.0 / np.sqrt(d)
    for i, h in enumerate(heads):
        sq, sk = slice(oq[i], oq[i + 1]), slice(ok[i], ok[i + 1])
        if lq[i] == 0:
            continue
        o_ref, lse_ref = A.forward(h["q"], h["k"], h["v"], h["qi"], h["ki"], h["qh"], h["kh"], scale)
        check_forward(o[sq], lse[sq], o_ref, lse_ref, dtype, f"varlen head {i}")
        if lk[i] == 0:
            assert np.all(dq[sq] == 0)
            continue
        g = A.backward(h["q"], h["k"], h["v"], h["do"], h["qi"], h["ki"], h["qh"], h["kh"], scale)
        check_grads([dq[sq], dk[sk], dv[sk]], g, dtype, f"varlen head {i}")
    for i in range(len(heads)):  # keys of heads with no queries get zero gradients
        if lq[i] == 0:
            assert np.all(dk[ok[i]:ok[i + 1]] == 0) and np.all(dv[ok[i]:ok[i + 1]] == 0)


@pytest.mark.parametrize("mode", ["qk", "hash"])
def test_varlen_equals_padded_layout(mode):
    """The padded layout (heads padded to the longest, padding queries at position -1 and padding
    keys at 2^31 - 1) gives the same real rows, bit for bit."""
    scfa = _lib()
    B, H, d, block = 1, 4, 64, 64
    lq, lk = [300, 1000, 129, 640], [280, 1000, 700, 64]
    heads = _heads(90, lq, lk, d, mode, 4, "bf16")
    note(f"[varlen vs padded] {mode}")
    mq, mk = max(lq), max(lk)
    cat = lambda key, dt=None: dev(np.concatenate([h[key] for h in heads]), dt)  # noqa: E731

    def pad(key, n, fill, dt=None):
        rows = []
        for h in heads:
            a = h[key]
            p = np.full((n - a.shape[0],) + a.shape[1:], fill, dtype=a.dtype)
            rows.append(np.concatenate([a, p]))
        return dev(np.stack(rows)[None], dt)

    qo, ko = dev(_offsets(lq)), dev(_offsets(lk))
    q, k, v, do = (cat(x, torch.bfloat16) for x in ("q", "k", "v", "do"))
    qi, ki = cat("qi"), cat("ki")
    qh, kh = (cat("qh"), cat("kh")) if mode == "hash" else (None, None)
    mt = dict(H=H, max_Tq=mq, max_Tk=mk)
    meta = scfa.block_meta_varlen(qo, ko, qi, ki, qh, kh, block=block, **mt)
    o, lse = scfa.attn_fwd_varlen(q, k, v, qo, ko, qi, ki, qh, kh, meta, block=block, **mt)
    dq, delta = scfa.attn_bwd_dq_varlen(q, k, v, o, lse, do, qo, ko, qi, ki, qh, kh, meta, block=block, **mt)
    dk, dv = scfa.attn_bwd_dkdv_varlen(q, k, v, lse, do, delta, qo, ko, qi, ki, qh, kh, meta, block=block, **mt)
    P = {x: pad(x, mq if x in ("q", "do") else mk, 0.0, torch.bfloat16) for x in ("q", "k", "v", "do")}
    pqi, pki = pad("qi", mq, -1), pad("ki", mk, 2**31 - 1)
    pqh, pkh = (pad("qh", mq, 0), pad("kh", mk, 0)) if mode == "hash" else (None, None)
    pm = scfa.block_meta(pqi, pki, pqh, pkh, block=block, with_cols=True, exact=True)
    o2, lse2 = scfa.attn_fwd_lists(P["q"], P["k"], P["v"], pqi, pki, pqh, pkh, pm, block=block)
    dq2, de2 = scfa.attn_bwd_dq_lists(P["q"], P["k"], P["v"], o2, lse2, P["do"], pqi, pki, pqh, pkh, pm, block=block)
    dk2, dv2 = scfa.attn_bwd_dkdv_lists(P["q"], P["k"], P["v"], lse2, P["do"], de2, pqi, pki, pqh, pkh, pm,
                                        block=block)
    torch.cuda.synchronize()
    oq, ok = _offsets(lq), _offsets(lk)
    for i in range(H):
        sq, sk = slice(oq[i], oq[i + 1]), slice(ok[i], ok[i + 1])
        assert torch.equal(o[sq], o2[0, i, : lq[i]]) and torch.equal(lse[sq], lse2[0, i, : lq[i]]), i
        assert torch.equal(dq[sq], dq2[0, i, : lq[i]]), i
        assert torch.equal(dk[sk], dk2[0, i, : lk[i]]) and torch.equal(dv[sk], dv2[0, i, : lk[i]]), i
