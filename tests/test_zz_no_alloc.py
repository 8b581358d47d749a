"""The allocation-free Hash-sparse forward against the workspace one.

scfa_hash_sparse_fwd_noalloc runs the same kernels as scfa_hash_sparse_fwd
with its scratch in a static per-GPU device array instead of a caller
workspace.  Two calls in a row through the raw C ABI (ctypes), the second
with a smaller input, so the second finds the first one's lists and segments
in the shared scratch: both must equal scfa_hash_sparse_fwd bit for bit.
"""

import ctypes

import numpy as np
import pytest

from gen import synthetic_case
from helpers import dev, note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _raw_noalloc(c_lib, q, k, v, qi, ki, qh, kh, block, scale):
    B, H, Tq, d = q.shape
    Tk = k.shape[2]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    fn = c_lib.scfa_hash_sparse_fwd_noalloc
    p = ctypes.c_void_p
    fn.argtypes = [p] * 9 + [ctypes.c_int] * 6 + [ctypes.c_float, ctypes.c_int, ctypes.c_uint, p]
    fn.restype = ctypes.c_int
    rc = fn(*(p(t.data_ptr()) for t in (q, k, v, qi, ki, qh, kh, o, lse)), B, H, Tq, Tk, d, block, scale,
            0 if q.dtype == torch.bfloat16 else 1, 0, p(torch.cuda.current_stream().cuda_stream))
    return rc, o, lse


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_forward_equals_workspace_forward(dtype):
    import sparse_causal_attention_amd as scfa
    from sparse_causal_attention_amd import _lib

    raw = ctypes.CDLL(_lib.LIB_PATH)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    cases = [dict(B=2, H=3, Tq=3000, Tk=2800, nb=8, block=64),
             dict(B=1, H=2, Tq=700, Tk=900, nb=5, block=128)]  # second call: smaller
    for i, kw in enumerate(cases):
        block = kw.pop("block")
        c = synthetic_case(70 + i, mode="hash", layout="grouped", dtype=dtype, **kw)
        note(f"[noalloc] call {i}: {kw} block={block} {dtype}")
        q, k, v = (dev(a, td) for a in (c.q, c.k, c.v))
        qi, ki, qh, kh = (dev(a) for a in (c.q_idx, c.k_idx, c.q_hash, c.k_hash))
        scale = 1.0 / np.sqrt(q.shape[-1])
        rc, o, lse = _raw_noalloc(raw, q, k, v, qi, ki, qh, kh, block, scale)
        assert rc == 0, raw.scfa_last_error
        o_ref, lse_ref = scfa.hash_sparse_fwd(q, k, v, qi, ki, qh, kh, block=block, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"call {i}: O differs"
        assert torch.equal(lse, lse_ref), f"call {i}: lse differs"
        # and through the binding
        o2, lse2 = scfa.hash_sparse_fwd_noalloc(q, k, v, qi, ki, qh, kh, block=block, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o2, o_ref) and torch.equal(lse2, lse_ref)
