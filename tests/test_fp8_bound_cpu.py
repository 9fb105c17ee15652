"""CPU check of the FP8 output bounds (parity_utils.fp8_bound) against a
float64 simulation of the weight rounding they cover, independent of the GPU.

The simulated kernel takes the exact weights of each row relative to a
running reference that may sit up to 2^8 below the row's maximum (the lazy
rescale), rounds them to E4M3 with the oracle's rounding (OCP E4M3, nearest,
ties to even), and forms the output either over the fp32-style exact
denominator (the call with LSE) or over the sum of the rounded weights
themselves (the call without LSE).  Scores are exact here (no product
accumulation error), so every simulated error must stay within the bound,
including a constructed row whose self-normalized output moves through its
denominator alone.
"""
import numpy as np
import pytest

import oracle as O
import oracle.fp8 as F8
from parity_utils import fp8_bound

BLK = 128


def _simulate(q, k, v, M, scale, shift_log2, self_norm):
    """float64 outputs of the simulated FP8 softmax over kept blocks."""
    N, D = q.shape
    out = np.full((N, D), np.nan)
    for r in range(M.shape[0]):
        rows = slice(r * BLK, min(N, (r + 1) * BLK))
        kept = np.nonzero(M[r])[0]
        if kept.size == 0:
            out[rows] = 0.0
            continue
        keys = np.concatenate([np.arange(c * BLK, min(N, (c + 1) * BLK)) for c in kept])
        s = (q[rows] @ k[keys].T) * scale
        w = np.exp(s - s.max(axis=1, keepdims=True)) * 2.0 ** shift_log2   # reference below the max
        qw = F8.e4m3_value(F8.e4m3_round(w))
        num = qw @ v[keys]
        den = qw.sum(axis=1, keepdims=True) if self_norm else w.sum(axis=1, keepdims=True)
        out[rows] = num / den
    return out


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("self_norm", [False, True])
def test_simulated_weight_rounding_within_bound(seed, self_norm):
    rng = np.random.default_rng(900 + seed)
    N, D = 3 * BLK + 37, 64
    q = rng.standard_normal((N, D)) * (1.0 + seed)          # peakier rows for larger seeds
    k = rng.standard_normal((N, D))
    v = rng.standard_normal((N, D)) + (2.0 if seed % 2 else 0.0)   # a mean offset: large |o|
    nB = -(-N // BLK)
    M = (rng.random((nB, nB)) < 0.6).astype(np.uint8)
    M[:, nB - 1] = 1
    scale = 1.0 / np.sqrt(D)
    bnd, _ = fp8_bound(q, k, v, M, BLK, scale, list(range(nB)), self_norm=self_norm)
    ref, _ = O.block_masked_attention(q, k, v, M, BLK, scale)
    for shift in (0, 3, 8):
        got = _simulate(q, k, v, M, scale, shift, self_norm)
        worst = float(np.max(np.abs(got - ref) / bnd))
        assert worst <= 1.0, (shift, worst)


def test_self_normalized_bound_needs_its_output_term():
    """Half of the keys carry weight 1 (exact in E4M3) and V rows of 10, the
    other half a weight just below 0.53125 (rounded down to 0.5, nearly 2^-4
    relative) and V rows of 0.  The self-normalized output moves with its
    denominator although every rounded weight multiplies a V row of 0 (an
    error of about 0.14 on outputs near 6.5), and the bound covers it."""
    D = 64
    N = BLK
    scale = 1.0 / np.sqrt(D)
    wb = 0.53125 - 1e-5
    s_keys = np.where(np.arange(N) < N // 2, 0.0, np.log(wb))
    q = np.zeros((N, D))
    q[:, 0] = 1.0
    k = np.zeros((N, D))
    k[:, 0] = s_keys / scale
    v = np.zeros((N, D))
    v[: N // 2] = 10.0
    M = np.ones((1, 1), np.uint8)
    ref, _ = O.block_masked_attention(q, k, v, M, BLK, scale)
    got = _simulate(q, k, v, M, scale, 0, True)
    err = np.abs(got - ref)
    bnd, _ = fp8_bound(q, k, v, M, BLK, scale, [0], self_norm=True)
    assert np.all(err <= bnd)
    assert np.all(err > 0.1)
    # the same output over the exact denominator moves by the rounded
    # weights' share only: Σ_B d_j v_j = 0 here
    got_exact_den = _simulate(q, k, v, M, scale, 0, False)
    assert np.max(np.abs(got_exact_den - ref)) < 1e-12
