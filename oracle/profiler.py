"""Online profiling: pick each head's mask by its error on sampled queries.

[SVG], "dynamic adaptive sparse strategy" (the three-step online profiling):
(1) at every inference step draw a small random set of query tokens (about 64);
(2) compute their attention under the spatial and under the temporal mask and
measure each result's error against dense attention; (3) give every head the
mask with the smaller error.

Readings:
* the sample set is supplied by the caller (64 distinct frame-major video
  token indices, one set shared by all heads of the call);
* error = squared L2 norm of (masked output - dense output), summed over the
  sampled rows and the head dimension (any normalisation common to both
  candidates leaves the choice unchanged);
* candidates are exactly {spatial, temporal}; a tie goes to spatial;
* each candidate is applied exactly as in the attention step: the spatial mask
  on frame-major blocks, the temporal mask on token-major blocks.
"""
import numpy as np

from .layout import token_major_index


def _admitted(i_rows, M, block_of_q, block_of_k):
    """bool [n, N]: key j admitted for query i under mask M (block-granular)."""
    return M[block_of_q[i_rows][:, None], block_of_k[None, :]] != 0


def _masked_rows(s, adm, v):
    """Softmax of each row of s over its admitted keys, times v (0 if none)."""
    out = np.zeros((s.shape[0], v.shape[1]))
    for n in range(s.shape[0]):
        a = adm[n]
        if not a.any():
            continue
        sa = s[n, a]
        e = np.exp(sa - sa.max())
        out[n] = (e @ v[a]) / e.sum()
    return out


def profile_heads(q, k, v, F, Hs, Ws, B, scale, idx, cand):
    """Head choice by sampled-query error.

    q, k, v: [H, N, D] frame-major (upcast to float64); idx: int [n_s];
    cand: uint8 [2, nB, nB] ([0] spatial on frame-major blocks, [1] temporal
    on token-major blocks).  Returns choice int32 [H] (0 spatial, 1 temporal)
    and err float64 [H, 2].
    """
    H, N, D = q.shape
    idx = np.asarray(idx, dtype=np.int64)
    p = token_major_index(F, Hs, Ws, N)
    blk_f = np.arange(N) // B            # frame-major block of every token
    blk_t = p // B                       # token-major block of every token
    adm_s = _admitted(idx, cand[0], blk_f, blk_f)
    adm_t = _admitted(idx, cand[1], blk_t, blk_t)
    everyone = np.ones_like(adm_s)
    err = np.zeros((H, 2))
    for h in range(H):
        qh = np.asarray(q[h], dtype=np.float64)
        kh = np.asarray(k[h], dtype=np.float64)
        vh = np.asarray(v[h], dtype=np.float64)
        s = (qh[idx] @ kh.T) * scale
        o_dense = _masked_rows(s, everyone, vh)
        for m, adm in enumerate((adm_s, adm_t)):
            d = _masked_rows(s, adm, vh) - o_dense
            err[h, m] = np.sum(d * d)
    choice = np.where(err[:, 0] <= err[:, 1], 0, 1).astype(np.int32)
    return choice, err


def profile_errors_decomposed(q, k, v, F, Hs, Ws, B, scale, idx, cand):
    """The same errors from per-class partial sums (float64).

    Every (query, key) pair falls in one of four classes: admitted by both
    masks, spatial only, temporal only, neither.  With Z_c = sum of exp(s - m)
    and U_c = sum of exp(s - m) v over class c, a mask's admitted set "in" and
    its complement "out" give Z = Z_in + Z_out and

        o_dense - o_mask = (Z_out / Z) * (U_out / Z_out - U_in / Z_in),

    an identity of exact arithmetic (o_mask = 0 when Z_in = 0; the difference
    is 0 when Z_out = 0).  Returns err float64 [H, 2].
    """
    H, N, D = q.shape
    idx = np.asarray(idx, dtype=np.int64)
    p = token_major_index(F, Hs, Ws, N)
    blk_f = np.arange(N) // B
    blk_t = p // B
    adm_s = _admitted(idx, cand[0], blk_f, blk_f)
    adm_t = _admitted(idx, cand[1], blk_t, blk_t)
    cls = np.where(adm_s, 0, 2) + np.where(adm_t, 0, 1)   # 0 both, 1 S only, 2 T only, 3 none
    err = np.zeros((H, 2))
    for h in range(H):
        qh = np.asarray(q[h], dtype=np.float64)
        kh = np.asarray(k[h], dtype=np.float64)
        vh = np.asarray(v[h], dtype=np.float64)
        s = (qh[idx] @ kh.T) * scale
        e = np.exp(s - s.max(axis=1, keepdims=True))
        Z = np.stack([np.where(cls == c, e, 0.0).sum(axis=1) for c in range(4)], axis=1)
        U = np.stack([np.where(cls == c, e, 0.0) @ vh for c in range(4)], axis=1)
        for m, inside in enumerate(((0, 1), (0, 2))):
            outside = tuple(c for c in range(4) if c not in inside)
            z_in, z_out = Z[:, inside].sum(axis=1), Z[:, outside].sum(axis=1)
            u_in, u_out = U[:, inside].sum(axis=1), U[:, outside].sum(axis=1)
            z = z_in + z_out
            diff = np.zeros_like(u_in)
            for n in range(len(idx)):
                if z_out[n] == 0.0:
                    continue
                if z_in[n] == 0.0:
                    diff[n] = (u_in[n] + u_out[n]) / z[n]
                else:
                    diff[n] = (z_out[n] / z[n]) * (u_out[n] / z_out[n] - u_in[n] / z_in[n])
            err[h, m] = np.sum(diff * diff)
    return err
