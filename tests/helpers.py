"""Shared pieces of the GPU parity tests: tolerances, comparisons, pipelines.

The GPU side calls only the library binding; the CPU side calls only the
oracle.  Both consume the same seeded arrays from ``gen``.
"""

from __future__ import annotations

import sys

import numpy as np

# Tolerances (forward: bf16 max abs 2e-2 and relative Frobenius 1e-2; fp32 max
# abs 1e-4; gradients: relative Frobenius 5e-2).  lse is gated at 1e-2 (bf16)
# and 1e-4 (fp32) absolute on rows with at least one admissible key.
FWD_BF16_MAX = 2e-2
FWD_BF16_REL = 1e-2
FWD_F32_MAX = 1e-4
GRAD_REL_BF16 = 5e-2
GRAD_REL_F32 = 1e-4
LSE_BF16 = 1e-2
LSE_F32 = 1e-4


def note(msg: str) -> None:
    """Name the case on stdout before a GPU step (flushed)."""
    print(msg, flush=True)
    sys.stdout.flush()


def rel_fro(got: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(np.asarray(got, dtype=np.float64) - ref)
    return float(num / den) if den > 0 else float(num)


def check_forward(o_gpu, lse_gpu, o_ref, lse_ref, dtype: str, what: str = "") -> None:
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), empty), f"{what}: empty-row pattern differs"
    assert np.all(o_gpu[empty] == 0.0), f"{what}: empty rows must be exactly 0"
    err = np.abs(o_gpu - o_ref).max() if o_ref.size else 0.0
    fin = ~empty
    lerr = np.abs(lse_gpu[fin] - lse_ref[fin]).max() if fin.any() else 0.0
    if dtype == "bf16":
        rf = rel_fro(o_gpu, o_ref)
        assert err <= FWD_BF16_MAX, f"{what}: max |dO| {err:.3e}"
        assert rf <= FWD_BF16_REL, f"{what}: rel Frobenius {rf:.3e}"
        assert lerr <= LSE_BF16, f"{what}: lse err {lerr:.3e}"
    else:
        assert err <= FWD_F32_MAX, f"{what}: max |dO| {err:.3e}"
        assert lerr <= LSE_F32, f"{what}: lse err {lerr:.3e}"


def check_grads(got, ref, dtype: str, what: str = "") -> None:
    tol = GRAD_REL_BF16 if dtype == "bf16" else GRAD_REL_F32
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        e = rel_fro(g, r)
        assert e <= tol, f"{what}: {name} rel Frobenius {e:.3e} > {tol}"


def to_np(t):
    import torch

    return t.detach().to("cpu", torch.float32).numpy() if t.is_floating_point() else t.detach().cpu().numpy()


def dev(a, dtype=None):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()
