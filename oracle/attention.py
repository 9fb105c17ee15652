"""Softmax attention, dense and block-masked, in float64.

Dense attention is softmax(q k^T / sqrt(D)) v per head, not causal ([VDA]
section 2.1 gives the formula; [SparsePR] section 2.1 the same computation on
[batch, heads, seq, dim] tensors).  Block-masked attention is the same
computation restricted, for each query block, to the keys of the key blocks the
mask keeps ([CalibAtt] sections 2.2 and 3.3: whole 128x128 blocks are kept or
skipped).  A query block whose mask row is empty has output 0 and
log-sum-exp -inf (reading: the pages never produce one; it arises only for the
non-anchor rows of row-repetitive heads, which are overwritten).
"""
import numpy as np

from .layout import to_token_major, to_frame_major


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """o [n, D] and natural-log lse [n] of softmax(q k^T * scale) v, float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = (q @ k.T) * scale
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    o = (e @ v) / z
    lse = m[:, 0] + np.log(z[:, 0])
    return o, lse


def block_masked_attention(q, k, v, M, B: int, scale: float, qblocks=None):
    """Block-masked attention of one head in the mask's own layout.

    q, k, v: [N, D] (any float dtype, upcast to float64); M: uint8 [nQB, nKB];
    qblocks: query blocks to compute (default all).  Returns o [N, D] and lse [N]
    as float64; rows of query blocks not computed are NaN.
    """
    N, D = q.shape
    o = np.full((N, D), np.nan)
    lse = np.full(N, np.nan)
    nQB = M.shape[0]
    qblocks = range(nQB) if qblocks is None else qblocks
    for r in qblocks:
        rows = slice(r * B, min(N, (r + 1) * B))
        kept = np.nonzero(M[r])[0]
        if kept.size == 0:
            o[rows] = 0.0
            lse[rows] = -np.inf
            continue
        keys = np.concatenate([np.arange(c * B, min(N, (c + 1) * B)) for c in kept])
        o[rows], lse[rows] = dense_attention(q[rows], k[keys], v[keys], scale)
    return o, lse


def head_attention(q, k, v, M, layout: int, F: int, Hs: int, Ws: int, B: int,
                   scale: float, qblocks=None):
    """Attention of one head whose mask M is defined in `layout`.

    layout 0: frame-major (mask blocks are frame-major blocks); layout 1:
    token-major ([SVG], "Layout Transformation"): q, k, v are permuted to
    token-major, attended there, and the output is permuted back.  qblocks are
    block ids in the mask's layout.  Returns frame-major o [N, D], lse [N].
    """
    if layout == 0:
        return block_masked_attention(q, k, v, M, B, scale, qblocks)
    qp, kp, vp = (to_token_major(np.asarray(t, dtype=np.float64), F, Hs, Ws) for t in (q, k, v))
    op, lsep = block_masked_attention(qp, kp, vp, M, B, scale, qblocks)
    return to_frame_major(op, F, Hs, Ws), to_frame_major(lsep[:, None], F, Hs, Ws)[:, 0]
