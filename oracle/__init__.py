"""CPU oracle for sparse causal flash attention (SCFA).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``sparse_causal_attention_amd``) never imports it, shares no code with it and
never falls back to it.

The oracle is the plain definition of what SCFA computes, evaluated in float64
from the exact values the GPU sees (bf16 inputs widened without rounding):

* ``attention``: the explicit element mask (original-position causality, and
  bucket equality in Hash-sparse mode) followed by dense masked softmax
  attention, its log-sum-exp, and analytic gradients.
* ``blocks``: per-block min/max of positions and bucket ids, the tile liveness
  and mask-free predicates, and the per-row / per-column live-tile lists,
  all by brute force over every block pair.
* ``coverage``: the share of bucket collisions (admissible pairs) a chunked
  within-bucket approximation visits, against SCFA's exact mask.
* ``rows``: gathering rows into compact / reordered tensors and scattering
  results back to their original rows.
* ``lsh``: the random-rotation LSH bucket (first maximum of ``[xR, -xR]``)
  with float64 accumulation in increasing coordinate order, and the stable
  ordering of tokens by (bucket, original position).

Citations name the deep-paper.org summary of arXiv 2306.01160, "Faster Causal
Attention Over Large Sequences Through Sparse Flash Attention" (page title
"超越 FlashAttention：利用动态稀疏性让 Transformer 再提速"), by section.

Pinning: every function is checked by ``tests/test_oracle_*.py`` against
library routines (torch's causal scaled-dot-product attention in float64 and
its autograd), brute force on tiny inputs, central finite differences,
integer-exact cases, closed forms and invariants.  Nothing here is
"parity unpinned".
"""

from . import attention, blocks, coverage, lsh, rows  # noqa: F401
