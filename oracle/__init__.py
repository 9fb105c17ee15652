"""fp64 CPU oracle of the block-sparse 3D attention path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports, calls or
links this package; only the tests, the smoke check and the bench's CPU
baseline leg use it.  It shares no code with the HIP path: it is plain NumPy
written from the pages' definitions, slow and obviously correct.

Sources cited in the modules:
  [SVG]      Sparse VideoGen article (m.jxzklqfsx.com/article/815093)
  [CalibAtt] calibrated sparse attention article (lpnh.cn/news/568491)
  [VDA]      video-diffusion acceleration survey (wmrh.cn/news/48564)
  [SparsePR] SparsePR tutorial (lqnn.cn/news/72918)
  RMSNorm: Zhang & Sennrich, "Root Mean Square Layer Normalization" (2019)
  RoPE:    Su et al., "RoFormer: Enhanced Transformer with Rotary Position
           Embedding" (2021)
  E4M3:    Open Compute Project, "OCP 8-bit Floating Point Specification
           (OFP8)" (2023)

Every function here is pinned by a CPU test to facts other than itself; none is
"parity unpinned".
"""
from .layout import token_major_index, to_token_major, to_frame_major
from .masks import (
    block_of_layout, spatial_block_mask, temporal_block_mask, apply_text_rule,
    online_candidate_masks, anchor_rows, anchor_query_blocks, restrict_to_anchor_blocks,
)
from .attention import dense_attention, block_masked_attention, head_attention
from .encode import encode_masks, decode_masks, iv_capacity
from .profiler import profile_heads, profile_errors_decomposed
from .calibrate import calibrate_row, calibrate_mask, block_energy, eps_schedule, aggregate_masks
from .broadcast import row_broadcast, row_patterns, row_similarity, is_row_repetitive
from .flops import kept_pairs, algorithmic_flops
from .norm_rope import rms_norm, rope_angles, rope_rotate, qk_norm_rope
from .fp8 import e4m3_value, e4m3_round, head_scale, quantize_head, vt8_key_order, vt8_blocks

__all__ = [
    "token_major_index", "to_token_major", "to_frame_major",
    "block_of_layout", "spatial_block_mask", "temporal_block_mask", "apply_text_rule",
    "online_candidate_masks", "anchor_rows", "anchor_query_blocks", "restrict_to_anchor_blocks",
    "dense_attention", "block_masked_attention", "head_attention",
    "encode_masks", "decode_masks", "iv_capacity",
    "profile_heads", "profile_errors_decomposed",
    "calibrate_row", "calibrate_mask", "block_energy", "eps_schedule", "aggregate_masks", "row_broadcast", "row_patterns", "row_similarity", "is_row_repetitive",
    "kept_pairs", "algorithmic_flops",
    "rms_norm", "rope_angles", "rope_rotate", "qk_norm_rope",
    "e4m3_value", "e4m3_round", "head_scale", "quantize_head", "vt8_key_order", "vt8_blocks",
]
