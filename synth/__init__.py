"""Seeded synthetic inputs shared by the oracle-side tests and the HIP path.

This package holds workload shapes and random-number recipes only: it computes
no attention, no mask, no permutation and no encoding.  Both the oracle and the
GPU path consume exactly the tensors produced here, so the two sides never
share any of the method's arithmetic.
"""
from .configs import CONFIGS, Workload, get_workload
from .generate import (
    head_classes,
    gen_head_qkv,
    gen_qkv,
    sample_query_idx,
    energy_matrix,
    repetitive_heads,
    to_bf16,
    gen_projection_rows,
    gen_norm_weight,
)

__all__ = [
    "CONFIGS", "Workload", "get_workload", "head_classes", "gen_head_qkv",
    "gen_qkv", "sample_query_idx", "energy_matrix", "repetitive_heads", "to_bf16",
    "gen_projection_rows", "gen_norm_weight",
]
