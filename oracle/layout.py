"""Frame-major <-> token-major layout ([SVG], "Layout Transformation + Kernel").

Frame-major storage keeps all tokens of one frame together, so the tokens at
one spatial position in different frames lie S = Hs*Ws rows apart.  The
token-major layout is the transpose of the (frame, position) grid: the F copies
of one position become one contiguous run.

Reading (the pages do not print a formula): video token i = f*S + s (s = y*Ws + x)
moves to p(i) = s*F + f; appended text tokens (i >= F*S) keep their index.
"""
import numpy as np


def token_major_index(F: int, Hs: int, Ws: int, N: int) -> np.ndarray:
    """p[i] = token-major position of frame-major token i, int64 [N]."""
    S = Hs * Ws
    p = np.arange(N, dtype=np.int64)
    i = np.arange(F * S, dtype=np.int64)
    f, s = np.divmod(i, S)
    p[: F * S] = s * F + f
    return p


def to_token_major(x: np.ndarray, F: int, Hs: int, Ws: int) -> np.ndarray:
    """y[..., p(i), :] = x[..., i, :] over the token axis (second to last)."""
    N = x.shape[-2]
    p = token_major_index(F, Hs, Ws, N)
    y = np.empty_like(x)
    y[..., p, :] = x
    return y


def to_frame_major(y: np.ndarray, F: int, Hs: int, Ws: int) -> np.ndarray:
    """Inverse of to_token_major: x[..., i, :] = y[..., p(i), :]."""
    N = y.shape[-2]
    p = token_major_index(F, Hs, Ws, N)
    return y[..., p, :].copy()
