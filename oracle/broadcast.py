"""Row broadcast of row-repetitive heads ([CalibAtt] section 3.2).

Some heads attend in nearly the same way from every row of a frame; for them
only k equally spaced anchor rows per frame are computed and each other row
reuses the result of its anchor, saving up to 1 - k/H of the work for H rows
per frame.

A head is taken as row-repetitive when the average cosine similarity between
the attention patterns of the rows of a frame exceeds gamma = 0.87.

Readings: a "row" is one latent image row (Ws tokens) of a frame; anchors are
band centres (see masks.anchor_rows); the output of token (f, y, x) becomes the
output of token (f, anchor(y), x) of the same head.  Text tokens are untouched.
The attention pattern of row (f, y) is the sum over its Ws queries of their
dense softmax weights over all N keys (text keys included); the average is the
plain mean of the cosine over every frame and every pair of distinct rows of
that frame; "exceeds" is strict.
"""
import numpy as np

from .masks import anchor_rows


def row_broadcast(o: np.ndarray, F: int, Hs: int, Ws: int, k: int) -> np.ndarray:
    """o [N, D] of one head, frame-major; returns the broadcast copy."""
    out = o.copy()
    a = anchor_rows(Hs, k)
    S = Hs * Ws
    for f in range(F):
        for y in range(Hs):
            src = f * S + a[y] * Ws
            dst = f * S + y * Ws
            out[dst:dst + Ws] = o[src:src + Ws]
    return out


def row_patterns(q: np.ndarray, k: np.ndarray, scale: float, F: int, Hs: int, Ws: int) -> np.ndarray:
    """float64 [F*Hs, N]: summed softmax weights of the queries of each latent row."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    A = np.zeros((F * Hs, k.shape[0]))
    for r in range(F * Hs):
        s = (q[r * Ws:(r + 1) * Ws] @ k.T) * scale
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        A[r] = p.sum(axis=0)
    return A


def row_similarity(q, k, scale: float, F: int, Hs: int, Ws: int) -> float:
    """Mean cosine similarity of the attention patterns of the rows of a frame."""
    A = row_patterns(q, k, scale, F, Hs, Ws)
    total, pairs = 0.0, 0
    for f in range(F):
        for y in range(Hs):
            for z in range(y + 1, Hs):
                a, b = A[f * Hs + y], A[f * Hs + z]
                total += float(a @ b) / float(np.sqrt((a @ a) * (b @ b)))
                pairs += 1
    return total / pairs


def is_row_repetitive(score: float, gamma: float = 0.87) -> bool:
    return score > gamma
