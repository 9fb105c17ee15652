"""Pins of the oracle's QK-Norm (RMS normalisation) and 3D rotary embedding
(CPU only): closed forms, invariants, a hand-worked case, and special cases
that reduce to NumPy's complex arithmetic."""
import json
import os

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


def test_rms_norm_unit_rms_and_scale_invariance():
    x = _rng(1).standard_normal((5, 3, 16)) * 3.0
    y = O.rms_norm(x, None, 0.0, "head")
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-12)
    np.testing.assert_allclose(O.rms_norm(7.5 * x, None, 0.0, "head"), y, rtol=1e-12)
    yr = O.rms_norm(x, None, 0.0, "row")
    np.testing.assert_allclose(np.sqrt(np.mean(yr * yr, axis=(-2, -1))), 1.0, rtol=1e-12)
    # the row form does not equalise heads of different size, the head form does
    x2 = x.copy()
    x2[:, 0] *= 10.0
    yr2 = O.rms_norm(x2, None, 0.0, "row")
    assert np.mean(yr2[:, 0] ** 2) > 10 * np.mean(yr2[:, 1] ** 2)
    np.testing.assert_allclose(O.rms_norm(x2, None, 0.0, "head"), y, rtol=1e-12)


def test_rms_norm_hand_case_gamma_eps():
    # (3, 4): mean square 12.5; with eps = 3.5 the divisor is sqrt(16) = 4
    x = np.array([[[3.0, 4.0]]])
    np.testing.assert_allclose(O.rms_norm(x, [2.0, -1.0], 3.5, "head"), [[[1.5, -1.0]]], rtol=1e-15)
    # a single head: "row" and "head" agree, gamma laid out per channel
    g = np.array([0.5, 2.0])
    np.testing.assert_allclose(O.rms_norm(x, g, 0.0, "row"), O.rms_norm(x, g, 0.0, "head"), rtol=1e-15)


def test_rope_hand_case():
    g = json.load(open(os.path.join(GOLD, "rope_hand_case.json")))
    a = O.rope_angles(g["F"], g["Hs"], g["Ws"], g["N"], g["d_axes"], g["theta"])
    np.testing.assert_allclose(a[g["token"]], g["angles"], rtol=1e-14)
    assert np.all(a[g["text_token"]] == 0.0)
    assert np.all(a[0] == 0.0)  # grid origin
    # pair (1, 0) turned by phi lands on (cos phi, sin phi): the sign convention
    x = np.zeros((g["N"], 12))
    x[:, 0::2] = 1.0
    y = O.rope_rotate(x, a)
    np.testing.assert_allclose(y[g["token"], 0::2], np.cos(g["angles"]), rtol=1e-14)
    np.testing.assert_allclose(y[g["token"], 1::2], np.sin(g["angles"]), rtol=1e-14)


def test_rope_is_complex_multiplication_and_keeps_pair_norms():
    F, Hs, Ws, N = 3, 4, 5, 70
    d_axes, theta = (8, 12, 12), 10000.0
    x = _rng(2).standard_normal((2, N, 32))
    a = O.rope_angles(F, Hs, Ws, N, d_axes, theta)
    y = O.rope_rotate(x, a)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * a)
    np.testing.assert_allclose(y[..., 0::2], z.real, atol=1e-13)
    np.testing.assert_allclose(y[..., 1::2], z.imag, atol=1e-13)
    np.testing.assert_allclose(np.hypot(y[..., 0::2], y[..., 1::2]), np.hypot(x[..., 0::2], x[..., 1::2]),
                               rtol=1e-13)


def test_rope_axis_runs():
    F, Hs, Ws = 3, 4, 5
    S = Hs * Ws
    d_axes = (8, 12, 12)
    a = O.rope_angles(F, Hs, Ws, F * S, d_axes, 10000.0)
    nz = lambda t: np.nonzero(a[t])[0].tolist()
    assert nz(1 * S) == list(range(0, 4))            # frame 1, (0, 0)
    assert nz(1 * Ws) == list(range(4, 10))          # frame 0, row 1
    assert nz(1) == list(range(10, 16))              # frame 0, column 1
    # frequencies fall geometrically inside a run, first one is 1 rad per step
    for t, lo, d in ((S, 0, 8), (Ws, 4, 12), (1, 10, 12)):
        run = a[t, lo:lo + d // 2]
        assert run[0] == 1.0
        np.testing.assert_allclose(run[1:] / run[:-1], 10000.0 ** (-2.0 / d), rtol=1e-13)


def test_rope_relative_position():
    """<R q, R k> depends on the grid offset of the two tokens only."""
    F, Hs, Ws = 4, 5, 6
    S = Hs * Ws
    N = F * S
    a = O.rope_angles(F, Hs, Ws, N, (8, 12, 12), 500.0)
    rng = _rng(3)
    q, k = rng.standard_normal(32), rng.standard_normal(32)
    X = np.zeros((N, 32))
    X[:] = q
    Rq = O.rope_rotate(X, a)
    X[:] = k
    Rk = O.rope_rotate(X, a)
    tok = lambda f, y, x: f * S + y * Ws + x
    d0 = Rq[tok(0, 1, 2)] @ Rk[tok(1, 3, 1)]
    d1 = Rq[tok(2, 2, 4)] @ Rk[tok(3, 4, 3)]   # both shifted by (2, 1, 2)
    assert abs(d0 - d1) < 1e-12
    d2 = Rq[tok(2, 2, 4)] @ Rk[tok(3, 4, 4)]   # a different offset
    assert abs(d0 - d2) > 1e-6


@pytest.mark.parametrize("norm", [None, "head", "row"])
def test_qk_norm_rope_layout_and_text(norm):
    F, Hs, Ws, text = 3, 2, 5, 7
    B, H, D = 2, 3, 16
    N = F * Hs * Ws + text
    x = _rng(4).standard_normal((B, N, H, D))
    gamma = _rng(5).uniform(0.5, 1.5, D if norm == "head" else H * D)
    rope = (4, 6, 6, 1000.0)
    lay = np.array([0, 1, 1, 0, 0, 1], np.int32)
    y = O.qk_norm_rope(x, F, Hs, Ws, norm, gamma, 1e-6, rope, lay)
    y0 = O.qk_norm_rope(x, F, Hs, Ws, norm, gamma, 1e-6, rope, None)
    assert y.shape == (B, H, N, D)
    for bh in range(B * H):
        b, h = divmod(bh, H)
        want = O.to_token_major(y0[b, h], F, Hs, Ws) if lay[bh] else y0[b, h]
        np.testing.assert_array_equal(y[b, h], want)
    # text rows are normalised (or copied) but never rotated
    base = O.rms_norm(x, gamma, 1e-6, norm) if norm else x
    np.testing.assert_allclose(y0[:, :, F * Hs * Ws:], np.transpose(base, (0, 2, 1, 3))[:, :, F * Hs * Ws:],
                               rtol=1e-14)
    # without norm and rope the call is a transpose
    np.testing.assert_array_equal(O.qk_norm_rope(x, F, Hs, Ws, None), np.transpose(x, (0, 2, 1, 3)))
