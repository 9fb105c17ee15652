"""Block masks of the two head types and of the text tokens.

A mask is a uint8 array [nQB, nKB]: entry 1 keeps the whole block pair (query
block r, key block c), 0 skips it.  Decisions are per block, matching the
tiled kernel ([CalibAtt] section 2.2 decides sparsity on 128x128 blocks); every
token pair inside a kept block is computed.

* Spatial ([SVG], "Spatial Head"): a head that looks at tokens of the same and
  of the adjacent frames.  Blocks are taken in frame-major order; the pair is
  kept when some video token of the query block and some video token of the key
  block are at most one frame apart.  Frames need not align with blocks.
* Temporal ([SVG], "Temporal Head"): a head that looks at the same position in
  other frames, a pattern of constant stride.  In token-major order those
  tokens are contiguous, so the mask is a band of half-width w around the
  block diagonal.
* Text tokens (appended after the video, never permuted): every key block that
  holds a text token is kept in every row, and every query block that holds a
  text token keeps every key block.
"""
import numpy as np


def n_blocks(N: int, B: int) -> int:
    return -(-N // B)


def block_of_layout(N: int, B: int) -> np.ndarray:
    """Block id of every position of a layout, int64 [N]."""
    return np.arange(N, dtype=np.int64) // B


def _frames_per_block(F: int, S: int, N: int, B: int) -> np.ndarray:
    """bool [nB, F]: frame f has a video token in frame-major block b."""
    nB = n_blocks(N, B)
    out = np.zeros((nB, F), dtype=bool)
    i = np.arange(F * S)
    out[i // B, i // S] = True
    return out


def apply_text_rule(M: np.ndarray, N_video: int, N: int, B: int) -> np.ndarray:
    """Keep every block pair whose query or key block holds a text token."""
    M = M.copy()
    nB = n_blocks(N, B)
    has_text = np.array([min(N, (b + 1) * B) > N_video for b in range(nB)])
    M[:, has_text] = 1
    M[has_text, :] = 1
    return M


def spatial_block_mask(F: int, Hs: int, Ws: int, N: int, B: int) -> np.ndarray:
    """Frame-major block mask of a spatial head (+/-1 frame), uint8 [nB, nB]."""
    S = Hs * Ws
    fr = _frames_per_block(F, S, N, B)
    near = fr.copy()                      # frames within one of a query block's frames
    near[:, 1:] |= fr[:, :-1]
    near[:, :-1] |= fr[:, 1:]
    M = (near.astype(np.int64) @ fr.T.astype(np.int64)) > 0
    return apply_text_rule(M.astype(np.uint8), F * S, N, B)


def temporal_block_mask(F: int, Hs: int, Ws: int, N: int, B: int, w: int) -> np.ndarray:
    """Token-major block mask of a temporal head (|r - c| <= w), uint8 [nB, nB]."""
    nB = n_blocks(N, B)
    r = np.arange(nB)
    M = (np.abs(r[:, None] - r[None, :]) <= w).astype(np.uint8)
    return apply_text_rule(M, F * Hs * Ws, N, B)


def online_candidate_masks(F, Hs, Ws, N, B, w) -> np.ndarray:
    """The two per-shape candidates, uint8 [2, nB, nB]: [0] spatial, [1] temporal."""
    return np.stack([spatial_block_mask(F, Hs, Ws, N, B),
                     temporal_block_mask(F, Hs, Ws, N, B, w)])


def anchor_rows(Hs: int, k: int) -> np.ndarray:
    """k equally spaced anchor rows of a frame ([CalibAtt] section 3.2).

    Reading: the rows are split into k equal bands and each band's centre row
    is its anchor, a_j = floor((2j+1)*Hs / (2k)); row y belongs to band
    floor(y*k / Hs).  Returns anchor_of_row, int64 [Hs].
    """
    y = np.arange(Hs)
    j = (y * k) // Hs
    return ((2 * j + 1) * Hs) // (2 * k)


def anchor_query_blocks(F: int, Hs: int, Ws: int, N: int, B: int, k: int) -> np.ndarray:
    """bool [nB]: frame-major query block holds at least one anchor-row video token."""
    S = Hs * Ws
    anchors = np.unique(anchor_rows(Hs, k))
    i = np.arange(F * S)
    y = (i % S) // Ws
    is_anchor = np.isin(y, anchors)
    out = np.zeros(n_blocks(N, B), dtype=bool)
    out[i[is_anchor] // B] = True
    return out


def restrict_to_anchor_blocks(M: np.ndarray, F, Hs, Ws, N, B, k) -> np.ndarray:
    """Empty the mask rows of query blocks that hold no anchor token."""
    M = M.copy()
    M[~anchor_query_blocks(F, Hs, Ws, N, B, k)] = 0
    return M
