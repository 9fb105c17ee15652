"""QK-Norm and 3D rotary position embedding of the query / key rows, the step
just before the attention ([SVG], "Layout Transformation + Kernel": the
custom QK-Norm and RoPE kernels, both measured against PyTorch).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The page names the two operations and their speed-ups but gives no formula.
The plainest readings, used here and listed with the others in the design
notes:

* QK-Norm is RMS normalisation (Zhang & Sennrich, "Root Mean Square Layer
  Normalization", 2019): y = x / sqrt(mean(x^2) + eps) * gamma, with the mean
  taken either over one head's D channels ("head", gamma of length D shared by
  the heads) or over the whole projection row of H*D channels ("row", gamma
  of length H*D).  No mean is subtracted.
* RoPE is the rotary embedding of RoFormer (Su et al., 2021) extended to the
  video grid: the D channels are cut into three runs of d_f, d_y and d_x
  channels for the frame, row and column of the token; in a run of length d,
  channel pair (2i, 2i+1) is turned by the angle pos * theta^(-2i/d), as the
  point x_{2i} + i x_{2i+1} of the complex plane.  Text tokens appended after
  the F*Hs*Ws video tokens have no grid position and are not rotated.
* The input is the projection output [B, N, H, D] in frame-major token order;
  the output is [B, H, N, D], each head written in its own layout (frame-major,
  or token-major: video token f*S + s at row s*F + f).
"""
import numpy as np

from .layout import token_major_index


def rms_norm(x: np.ndarray, gamma, eps: float, span: str) -> np.ndarray:
    """RMS normalisation of x [..., H, D] over "head" (D) or "row" (H*D); gamma
    None means all ones.  fp64."""
    x = np.asarray(x, dtype=np.float64)
    H, D = x.shape[-2:]
    if span == "head":
        ms = np.mean(x * x, axis=-1, keepdims=True)
        g = np.ones(D) if gamma is None else np.asarray(gamma, np.float64).reshape(D)
    elif span == "row":
        ms = np.mean(x * x, axis=(-2, -1), keepdims=True)
        g = np.ones((H, D)) if gamma is None else np.asarray(gamma, np.float64).reshape(H, D)
    else:
        raise ValueError(span)
    return x / np.sqrt(ms + eps) * g


def rope_angles(F: int, Hs: int, Ws: int, N: int, d_axes, theta: float) -> np.ndarray:
    """Rotation angle of every channel pair of every token, fp64 [N, D/2].

    Token n < F*Hs*Ws sits at frame f = n // S, row y = (n % S) // Ws, column
    x = n % Ws (S = Hs*Ws).  Pairs [0, d_f/2) turn with f, the next d_y/2 with
    y, the last d_x/2 with x; pair i of a run of d channels has frequency
    theta^(-2i/d).  Text tokens get angle 0."""
    d_f, d_y, d_x = d_axes
    S = Hs * Ws
    Nv = F * S
    n = np.arange(N)
    f, s = np.divmod(n, S)
    y, xcol = np.divmod(s, Ws)
    ang = []
    for pos, d in ((f, d_f), (y, d_y), (xcol, d_x)):
        freq = theta ** (-2.0 * np.arange(d // 2) / d)
        ang.append(pos[:, None].astype(np.float64) * freq[None, :])
    a = np.concatenate(ang, axis=1)
    a[n >= Nv] = 0.0
    return a


def rope_rotate(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Turn channel pairs (2i, 2i+1) of x [..., N, D] by angles [N, D/2]."""
    x = np.asarray(x, dtype=np.float64)
    a, b = x[..., 0::2], x[..., 1::2]
    c, s = np.cos(angles), np.sin(angles)
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def qk_norm_rope(x: np.ndarray, F: int, Hs: int, Ws: int, norm: str = "head", gamma=None,
                 eps: float = 1e-6, rope=None, head_layout=None) -> np.ndarray:
    """[B, N, H, D] projection rows -> [B, H, N, D] attention input, fp64.

    norm: None, "head" or "row"; rope: None or (d_f, d_y, d_x, theta);
    head_layout: None or int [B*H], nonzero = that head's rows token-major."""
    x = np.asarray(x, dtype=np.float64)
    B, N, H, D = x.shape
    y = rms_norm(x, gamma, eps, norm) if norm is not None else x.copy()
    y = np.transpose(y, (0, 2, 1, 3))  # [B, H, N, D]
    if rope is not None:
        d_f, d_y, d_x, theta = rope
        y = rope_rotate(y, rope_angles(F, Hs, Ws, N, (d_f, d_y, d_x), theta))
    out = np.array(y)
    if head_layout is not None:
        p = token_major_index(F, Hs, Ws, N)
        lay = np.asarray(head_layout).reshape(B, H)
        for b in range(B):
            for h in range(H):
                if lay[b, h] != 0:
                    out[b, h, p, :] = y[b, h]
    return out
