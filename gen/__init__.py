"""Seeded synthetic inputs for the sparse causal attention workloads.

This package only draws random numbers: Gaussian Q/K/V/dO tensors, Gaussian
LSH rotation matrices and uniform keep-sets of token positions.  It holds none
of the method's arithmetic (no hashing, sorting, masking, block tests or
attention); both the CPU oracle and the GPU path consume the arrays it returns.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    HeadInputs,
    bf16_round,
    custom_workload,
    head_inputs,
    lsh_rotation,
    keep_set,
    SyntheticCase,
    synthetic_case,
)
