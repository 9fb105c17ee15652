"""Attention-layer drivers built from the C ABI calls.

OnlineSparseAttention follows the Sparse VideoGen flow ([SVG], online
profiling and layout transformation): profile the heads on sampled queries,
move the temporal heads to token-major order, run block-sparse attention with
each head's chosen mask, move those heads' outputs back.  The head choice
stays on the device: the same `choice` array selects the permuted heads, the
mask and the layout, so nothing returns to the host inside a call.

StaticSparseAttention follows the calibrated-mask flow ([CalibAtt] sections
3.1-3.3): one fixed encoded mask per head, and anchor-row broadcast for the
row-repetitive heads.
"""
import math

import numpy as np
import torch

from .ops import (Shape, EncodedMasks, svg_build_masks, svg_encode_mask, svg_permute,
                  svg_profile_workspace_bytes, svg_profile_heads, svg_attn_workspace_bytes,
                  svg_block_sparse_attn, svg_row_broadcast, svg_restrict_anchor_rows,
                  svg_qk_norm_rope, svg_vt_bytes, svg_prepare_kv)


class OnlineSparseAttention:
    """fused_layout (128-token blocks): after the head choice one layout pass
    (svg_prepare_kv) writes the temporal heads' K token-major and every head's
    V block-transposed in its layout; the attention reads the temporal heads'
    Q rows and writes their O rows through the permutation, so no other move
    and no inverse move follow.  Otherwise (64-token blocks) q, k, v of the
    temporal heads go through svg_permute and op back."""

    def __init__(self, s: Shape, band_w: int, scale: float = None, n_samples: int = 64,
                 device="cuda", fused_layout: bool = None):
        self.s = s
        self.scale = scale if scale is not None else 1.0 / math.sqrt(s.D)
        self.n_samples = n_samples
        self.dense_masks = svg_build_masks(s, band_w, device=device)
        self.cand = svg_encode_mask(self.dense_masks)
        self.workspace = torch.empty(svg_profile_workspace_bytes(s, n_samples), dtype=torch.uint8,
                                     device=device)
        self.choice = torch.zeros(s.B * s.H, dtype=torch.int32, device=device)
        self.err = torch.zeros((s.B * s.H, 2), dtype=torch.float32, device=device)
        self.fused_layout = (s.block == 128) if fused_layout is None else fused_layout
        shape = (s.B, s.H, s.N, s.D)
        self.kp = torch.empty(shape, dtype=torch.bfloat16, device=device)
        self.qp, self.vp, self.op = (None, None, None) if self.fused_layout else (
            torch.empty(shape, dtype=torch.bfloat16, device=device) for _ in range(3))
        self.vt = (torch.empty(svg_vt_bytes(s) // 2, dtype=torch.bfloat16, device=device)
                   if self.fused_layout else None)
        self.attn_workspace = torch.empty(max(svg_attn_workspace_bytes(s, self.fused_layout), 1),
                                          dtype=torch.uint8, device=device)

    def prepare_inputs(self, xq, xk, xv, norm="row", gamma_q=None, gamma_k=None, eps=1e-6, rope=None,
                       out=None):
        """Attention inputs from the projection rows xq, xk, xv [B, N, H, D]
        (frame-major tokens): q and k RMS-normalised (norm = "head", "row" or
        None, weights gamma_q / gamma_k) and turned by the 3D rotary embedding
        rope = (d_f, d_y, d_x, theta) or not (None); v moved unchanged.  All
        three come out frame-major [B, H, N, D] (the profiler reads every head
        before the layouts are chosen).  out: optional (q, k, v) to fill."""
        q, k, v = out if out is not None else (None, None, None)
        q = svg_qk_norm_rope(xq, self.s, norm=norm, gamma=gamma_q, eps=eps, rope=rope, out=q)
        k = svg_qk_norm_rope(xk, self.s, norm=norm, gamma=gamma_k, eps=eps, rope=rope, out=k)
        v = svg_qk_norm_rope(xv, self.s, norm=None, rope=None, out=v)
        return q, k, v

    def profile(self, q, k, v, idx):
        return svg_profile_heads(q, k, v, self.s, self.scale, idx, self.cand, self.workspace,
                                 self.choice, self.err)

    def permute_inputs(self, q, k, v):
        """The layout step after the head choice: K token-major and every
        head's V^T blocks in one pass when fused, else svg_permute of q, k, v."""
        if self.fused_layout:
            svg_prepare_kv(k, v, self.s, head_layout=self.choice, kp=self.kp, vt=self.vt)
            return
        for x, y in ((q, self.qp), (k, self.kp), (v, self.vp)):
            svg_permute(x, self.s, self.choice, inverse=False, out=y)

    def attend(self, q, k, v, out=None, lse=False):
        return svg_block_sparse_attn(q, k, v, self.s, self.scale, self.cand,
                                     head_mask=self.choice, head_layout=self.choice,
                                     qp=self.qp, kp=self.kp, vp=self.vp, out=out,
                                     op=self.op, lse=lse, workspace=self.attn_workspace, vt=self.vt)

    def restore_output(self, out):
        """Frame-major output of the temporal heads (nothing to do when fused)."""
        if self.op is not None:
            svg_permute(self.op, self.s, self.choice, inverse=True, out=out)

    def __call__(self, q, k, v, idx, out=None, lse=False):
        self.profile(q, k, v, idx)
        self.permute_inputs(q, k, v)
        out, _, lse_t = self.attend(q, k, v, out=out, lse=lse)
        self.restore_output(out)
        return out, lse_t


class StaticSparseAttention:
    def __init__(self, s: Shape, dense_masks: torch.Tensor, repetitive: torch.Tensor = None,
                 k_anchors: int = 5, scale: float = None):
        """dense_masks: uint8 [H, nB, nB] (one mask per head, shared by every
        batch row); repetitive: int32 device flags of the row-repetitive heads,
        [H] or [B*H] with the same flags in every batch row (the mask of a head
        is restricted to its anchor rows once for all batch rows), or None."""
        self.s = s
        self.scale = scale if scale is not None else 1.0 / math.sqrt(s.D)
        self.k = k_anchors
        masks = dense_masks.clone()
        self.repetitive = None
        if repetitive is not None:
            if repetitive.numel() == s.H:
                flags = repetitive.reshape(s.H)
            elif repetitive.numel() == s.B * s.H:
                rows = repetitive.reshape(s.B, s.H)
                if not torch.equal(rows, rows[:1].expand_as(rows)):
                    raise ValueError("the masks are per head: the repetitive flags must be the same "
                                     "in every batch row")
                flags = rows[0]
            else:
                raise ValueError(f"repetitive must hold {s.H} or {s.B * s.H} flags")
            flags = flags.contiguous()
            svg_restrict_anchor_rows(masks, s, flags, k_anchors)
            self.repetitive = flags.repeat(s.B).contiguous()   # per (batch, head) for the broadcast
        self.masks = svg_encode_mask(masks)
        self.attn_workspace = torch.empty(max(svg_attn_workspace_bytes(s), 1), dtype=torch.uint8,
                                          device=dense_masks.device)

    def __call__(self, q, k, v, out=None, lse=False):
        out, _, lse_t = svg_block_sparse_attn(q, k, v, self.s, self.scale, self.masks, out=out,
                                              lse=lse, workspace=self.attn_workspace)
        if self.repetitive is not None:
            svg_row_broadcast(out, self.s, self.repetitive, self.k)
        return out, lse_t


def kept_pairs_per_mask(masks: EncodedMasks, N: int, block: int) -> np.ndarray:
    """(query, key) token pairs inside the kept blocks of each encoded mask,
    counted from the skip list (tokens past N excluded).  int64 [n_masks]."""
    rp = masks.row_ptr.cpu().numpy().astype(np.int64)
    iv = masks.iv[: int(rp[-1])].cpu().numpy().astype(np.int64)
    n_qb = masks.n_qb

    def tokens_upto(c):  # tokens in key blocks [0, c)
        return np.minimum(c * block, N)

    per_iv = tokens_upto(iv[:, 1]) - tokens_upto(iv[:, 0]) if len(iv) else np.zeros(0, np.int64)
    rows = np.repeat(np.arange(len(rp) - 1), np.diff(rp))
    row_keys = np.bincount(rows, weights=per_iv, minlength=len(rp) - 1).astype(np.int64)
    r = np.arange(n_qb)
    q_tokens = np.minimum((r + 1) * block, N) - r * block
    return (row_keys.reshape(masks.n_masks, n_qb) * q_tokens[None, :]).sum(axis=1)


def attention_flops(masks: EncodedMasks, head_mask, N: int, block: int, D: int) -> int:
    """Algorithmic FLOP of one block-sparse attention call: 4*D per kept
    (query, key) pair (one multiply-add each for q.k and p.v per head dim)."""
    pairs = kept_pairs_per_mask(masks, N, block)
    return int(sum(4 * D * int(pairs[m]) for m in head_mask))
