"""Row broadcast of row-repetitive heads ([CalibAtt] section 3.2).

Some heads attend in nearly the same way from every row of a frame; for them
only k equally spaced anchor rows per frame are computed and each other row
reuses the result of its anchor, saving up to 1 - k/H of the work for H rows
per frame.

Readings: a "row" is one latent image row (Ws tokens) of a frame; anchors are
band centres (see masks.anchor_rows); the output of token (f, y, x) becomes the
output of token (f, anchor(y), x) of the same head.  Text tokens are untouched.
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
