"""Workload definitions and seeded generators.

Every random stream is a NumPy ``Generator(PCG64)`` seeded by a
``SeedSequence`` whose entropy names the workload and the (batch, head) it
belongs to, so any head can be regenerated on its own:

* LSH rotation ``R_h``: ``SeedSequence([seed, 1, h])``, standard normal,
  float32, shape ``[d, n_buckets // 2]``; one matrix per head, shared by the
  batch and by Q and K.
* keep-sets: ``SeedSequence([seed, 2, b, h])``, ``choice(T, n_keep,
  replace=False)`` sorted ascending.  With independent Q and K drops the Q set
  is drawn first, then the K set, from the same stream.
* activations: ``SeedSequence([seed, 3, b, h])``, standard normal float32 in
  the order Q, K, V, dO; for bf16 workloads each value is rounded to the
  nearest bfloat16 (ties to even) so that the CPU and the GPU see identical
  numbers.

For the five named workloads ``seed`` is the workload number (1..5).
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and sparsity recipe of one synthetic workload."""

    name: str
    seed: int
    mode: str  # "qk" (token drop only), "hash" (LSH buckets), "hash_drop" (drop, then LSH)
    dtype: str  # "bf16" or "fp32"
    B: int
    H: int
    T: int  # original sequence length
    d: int
    block: int
    n_keep: int  # kept tokens per head (== T when nothing is dropped)
    n_buckets: Optional[int]  # None for QK-sparse
    train: bool  # forward + backward (draws dO)
    shared_keep: bool = True  # one keep-set for Q and K (else independent sets)
    n_keep_k: Optional[int] = None  # K keep count when the sets are independent

    @property
    def Tq(self) -> int:
        return self.n_keep

    @property
    def Tk(self) -> int:
        return self.n_keep if self.shared_keep else int(self.n_keep_k)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


def _kept(T: int, drop_fraction: float) -> int:
    return T - int(round(drop_fraction * T))


# The five workloads of the benchmark suite.  Keep counts: 256 - round(0.3*256)
# = 179; 8192 - round(0.3*8192) = 5734; 2**20 - 2**19 = 524288.
WORKLOADS = {
    1: Workload("qk_fwd_fp32_T256", 1, "qk", "fp32", 1, 1, 256, 64, 64, _kept(256, 0.3), None, False),
    2: Workload("hash_fwd_bf16_T8192_nb16", 2, "hash", "bf16", 1, 8, 8192, 64, 64, 8192, 16, False),
    3: Workload("qk_train_bf16_T8192_drop30", 3, "qk", "bf16", 4, 12, 8192, 64, 64, _kept(8192, 0.3), None, True),
    4: Workload("hash_train_bf16_T16384_nb32", 4, "hash", "bf16", 2, 12, 16384, 64, 64, 16384, 32, True),
    5: Workload("hash_drop50_fwd_bf16_T1M_nb256", 5, "hash_drop", "bf16", 1, 8, 1 << 20, 128, 128, 1 << 19, 256, False),
}


def custom_workload(
    *,
    seed: int,
    mode: str,
    B: int = 1,
    H: int = 1,
    T: int,
    d: int = 64,
    block: int = 64,
    dtype: str = "bf16",
    n_keep: Optional[int] = None,
    n_keep_k: Optional[int] = None,
    n_buckets: Optional[int] = None,
    train: bool = False,
) -> Workload:
    """A small workload for tests (ragged tails, odd sizes, independent drops)."""
    if n_keep is None:
        n_keep = T
    shared = n_keep_k is None
    return Workload(
        name=f"custom_s{seed}",
        seed=seed,
        mode=mode,
        dtype=dtype,
        B=B,
        H=H,
        T=T,
        d=d,
        block=block,
        n_keep=n_keep,
        n_buckets=n_buckets,
        train=train,
        shared_keep=shared,
        n_keep_k=n_keep_k,
    )


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    bits = (bits + 0x7FFF + lsb) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


def _rng(*entropy: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(entropy))))


def lsh_rotation(w: Workload, h: int) -> np.ndarray:
    """R_h: float32 [d, n_buckets/2] standard normal (shared by batch, Q and K)."""
    assert w.n_buckets is not None and w.n_buckets % 2 == 0
    return _rng(w.seed, 1, h).standard_normal((w.d, w.n_buckets // 2), dtype=np.float32)


def keep_set(w: Workload, b: int, h: int):
    """Kept original positions (int32, ascending) for Q and for K of one head.

    Returns ``(q_keep, k_keep)``; they are the same array for a shared set.
    With nothing dropped both are ``arange(T)``.
    """
    if w.n_keep == w.T and w.shared_keep:
        a = np.arange(w.T, dtype=np.int32)
        return a, a
    g = _rng(w.seed, 2, b, h)
    q = np.sort(g.choice(w.T, w.n_keep, replace=False)).astype(np.int32)
    if w.shared_keep:
        return q, q
    k = np.sort(g.choice(w.T, w.Tk, replace=False)).astype(np.int32)
    return q, k


@dataclasses.dataclass
class HeadInputs:
    """Inputs of one (b, h) in original token order (rows = kept tokens)."""

    q: np.ndarray  # [Tq, d] float32 (bf16-exact for bf16 workloads)
    k: np.ndarray  # [Tk, d]
    v: np.ndarray  # [Tk, d]
    do: Optional[np.ndarray]  # [Tq, d] upstream gradient, training workloads only
    q_pos: np.ndarray  # [Tq] int32 original positions, ascending
    k_pos: np.ndarray  # [Tk] int32


def head_inputs(w: Workload, b: int, h: int, *, with_do: Optional[bool] = None) -> HeadInputs:
    """Draw Q, K, V (and dO) for one head; rows follow ascending original position."""
    q_pos, k_pos = keep_set(w, b, h)
    g = _rng(w.seed, 3, b, h)
    q = g.standard_normal((w.Tq, w.d), dtype=np.float32)
    k = g.standard_normal((w.Tk, w.d), dtype=np.float32)
    v = g.standard_normal((w.Tk, w.d), dtype=np.float32)
    want_do = w.train if with_do is None else with_do
    do = g.standard_normal((w.Tq, w.d), dtype=np.float32) if want_do else None
    if w.dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
        if do is not None:
            do = bf16_round(do)
    return HeadInputs(q=q, k=k, v=v, do=do, q_pos=q_pos, k_pos=k_pos)


@dataclasses.dataclass
class SyntheticCase:
    """Arrays [B, H, ...] for a small attention case (float32 values, bf16-exact if bf16)."""

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray
    q_idx: Optional[np.ndarray]
    k_idx: Optional[np.ndarray]
    q_hash: Optional[np.ndarray]
    k_hash: Optional[np.ndarray]
    dtype: str


def _grouped(rng, T_orig, n, nb, layout):
    """n distinct positions of [0, T_orig) with random bucket ids in [0, nb).

    layout "grouped": rows listed bucket by bucket, positions ascending inside a
    bucket (the layout LSH reordering produces); "ascending": positions
    ascending; "shuffled": random row order.
    """
    pos = np.sort(rng.choice(T_orig, n, replace=False)).astype(np.int32)
    hs = rng.integers(0, nb, n).astype(np.int32) if nb else np.zeros(n, np.int32)
    if layout == "grouped":
        rows = np.concatenate([np.nonzero(hs == c)[0] for c in range(max(nb, 1))])
    elif layout == "shuffled":
        rows = rng.permutation(n)
    else:
        rows = np.arange(n)
    return pos[rows], hs[rows]


def synthetic_case(
    seed: int,
    *,
    B: int = 1,
    H: int = 1,
    Tq: int,
    Tk: int,
    d: int = 64,
    dtype: str = "bf16",
    mode: str = "qk",  # "dense", "qk" or "hash"
    nb: int = 0,
    layout: str = "ascending",
    shared: bool = False,
    T_orig: Optional[int] = None,
) -> SyntheticCase:
    """Seeded Gaussian Q/K/V/dO with random original positions and bucket ids.

    ``shared`` uses one position (and bucket) vector for Q and K (requires
    Tq == Tk).  Dense mode returns no positions (the library then uses row
    numbers).
    """
    g = _rng(seed, 4)
    if T_orig is None:
        T_orig = 2 * max(Tq, Tk, 1)
    q = g.standard_normal((B, H, Tq, d), dtype=np.float32)
    k = g.standard_normal((B, H, Tk, d), dtype=np.float32)
    v = g.standard_normal((B, H, Tk, d), dtype=np.float32)
    do = g.standard_normal((B, H, Tq, d), dtype=np.float32)
    if dtype == "bf16":
        q, k, v, do = (bf16_round(a) for a in (q, k, v, do))
    if mode == "dense":
        return SyntheticCase(q, k, v, do, None, None, None, None, dtype)
    qi = np.zeros((B, H, Tq), np.int32)
    ki = np.zeros((B, H, Tk), np.int32)
    qh = np.zeros((B, H, Tq), np.int32)
    kh = np.zeros((B, H, Tk), np.int32)
    nbk = nb if mode == "hash" else 0
    for b in range(B):
        for h in range(H):
            qi[b, h], qh[b, h] = _grouped(g, T_orig, Tq, nbk, layout)
            if shared:
                ki[b, h], kh[b, h] = qi[b, h], qh[b, h]
            else:
                ki[b, h], kh[b, h] = _grouped(g, T_orig, Tk, nbk, layout)
    if mode == "qk":
        return SyntheticCase(q, k, v, do, qi, ki, None, None, dtype)
    return SyntheticCase(q, k, v, do, qi, ki, qh, kh, dtype)
