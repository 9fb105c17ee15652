"""Block-sparse 3D attention for video diffusion transformers on MI355X (gfx950).

Spatial / temporal head masks, the frame-major <-> token-major layout
permutation, the fused QK-Norm + 3D RoPE step before the attention, sampled-query online head profiling and calibrated static masks
encoded as bitmap + skip list, all computed by the HIP kernels of libsvg.so
behind the C ABI in include/svg.h.  This package is the thin Python binding.
"""
from .ops import (
    Shape, EncodedMasks,
    svg_build_masks, svg_encode_iv_capacity, svg_encode_mask, svg_permute,
    svg_profile_workspace_bytes, svg_profile_heads, svg_attn_workspace_bytes,
    svg_block_sparse_attn, svg_row_broadcast, svg_restrict_anchor_rows, svg_calibrate_masks, svg_version,
    svg_block_energy, svg_aggregate_masks, svg_eps_schedule, svg_row_similarity,
    svg_row_similarity_workspace_bytes, svg_qk_norm_rope, svg_vt_bytes, svg_prepare_kv,
    svg_noalloc_scratch_bytes, svg_block_sparse_attn_noalloc,
    Fp8Operands, svg_fp8_vt_bytes, svg_quantize_fp8, svg_block_sparse_attn_fp8,
    svg_mfma_peak_probe,
)
from .layer import OnlineSparseAttention, StaticSparseAttention, attention_flops, kept_pairs_per_mask
from ._lib import SvgError, LIB_PATH

__all__ = [
    "Shape", "EncodedMasks", "svg_build_masks", "svg_encode_iv_capacity", "svg_encode_mask",
    "svg_permute", "svg_profile_workspace_bytes", "svg_profile_heads", "svg_attn_workspace_bytes",
    "svg_block_sparse_attn",
    "svg_row_broadcast", "svg_restrict_anchor_rows", "svg_calibrate_masks", "svg_version",
    "svg_block_energy", "svg_aggregate_masks", "svg_eps_schedule", "svg_row_similarity",
    "svg_row_similarity_workspace_bytes", "svg_qk_norm_rope", "svg_vt_bytes", "svg_prepare_kv",
    "svg_noalloc_scratch_bytes", "svg_block_sparse_attn_noalloc",
    "Fp8Operands", "svg_fp8_vt_bytes", "svg_quantize_fp8", "svg_block_sparse_attn_fp8",
    "svg_mfma_peak_probe",
    "OnlineSparseAttention", "StaticSparseAttention", "attention_flops", "kept_pairs_per_mask",
    "SvgError", "LIB_PATH",
]
