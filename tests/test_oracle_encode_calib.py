"""Pins of the oracle's mask encoding and energy-threshold calibration (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle as O
import synth as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _check_encoding(M):
    bm, rp, iv = O.encode_masks(M)
    n_masks, nQB, nKB = M.shape
    assert bm.shape == (n_masks, nQB, -(-nKB // 32)) and bm.dtype == np.uint32
    assert rp.shape == (n_masks * nQB + 1,) and rp[0] == 0 and rp[-1] == len(iv)
    fb, fi = O.decode_masks(bm, rp, iv, nKB)
    assert np.array_equal(fb, (M != 0).astype(np.uint8))
    assert np.array_equal(fi, (M != 0).astype(np.uint8))
    # padding bits are zero
    W = bm.shape[2]
    if nKB % 32:
        assert np.all(bm[:, :, W - 1] >> np.uint32(nKB % 32) == 0)
    for row in range(n_masks * nQB):
        seg = iv[rp[row]:rp[row + 1]]
        assert np.all(seg[:, 0] < seg[:, 1])
        assert np.all(seg[1:, 0] > seg[:-1, 1])           # disjoint and maximal
        pop = sum(bin(int(x)).count("1") for x in bm.reshape(-1, W)[row])
        assert pop == int(np.sum(seg[:, 1] - seg[:, 0]))
    assert len(iv) <= O.iv_capacity(n_masks, nQB, nKB)
    return bm, rp, iv


def test_hand_encoded_row():
    g = json.load(open(os.path.join(GOLD, "encode_small.json")))
    M = np.array(g["row"], np.uint8)[None, None]
    bm, rp, iv = _check_encoding(M)
    assert bm.ravel().tolist() == g["bitmap_words"]
    assert iv.tolist() == g["intervals"]


@pytest.mark.parametrize("shape,p", [((3, 17, 70), 0.5), ((2, 5, 64), 0.1), ((1, 40, 33), 0.9),
                                     ((2, 9, 32), 0.0), ((1, 3, 1), 1.0)])
def test_random_masks_roundtrip(shape, p):
    M = (np.random.default_rng(sum(shape)).random(shape) < p).astype(np.uint8)
    _check_encoding(M)


def test_alternating_row_reaches_capacity():
    nKB = 71
    M = np.zeros((2, 3, nKB), np.uint8)
    M[..., ::2] = 1
    bm, rp, iv = _check_encoding(M)
    assert len(iv) == O.iv_capacity(2, 3, nKB)


def test_bitmap_is_32x_smaller():
    # [CalibAtt] section 3.3: one bit per block instead of a 32-bit entry
    M = np.ones((1, 64, 128), np.uint8)
    bm, _, _ = O.encode_masks(M)
    assert M.size * 4 == 32 * bm.nbytes


def test_online_masks_sizes():
    w = S.get_workload("wan720p")
    M = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    bm, rp, iv = _check_encoding(M)
    assert bm.shape == (2, 591, 19)
    assert len(iv) == 2 * 591              # both masks are one interval per row


def test_calibrate_eps_one_keeps_all_positive():
    E = np.array([[3.0, 0.0, 1.0, 5.0, 2.0], [0.0, 0.0, 7.0, 0.0, 1.0]])
    M = O.calibrate_mask(E, 1.0)
    assert np.array_equal(M, (E > 0).astype(np.uint8))


def test_calibrate_tiny_eps_keeps_argmax():
    rng = np.random.default_rng(3)
    E = rng.random((20, 30))
    M = O.calibrate_mask(E, 1e-300)
    assert np.all(M.sum(axis=1) == 1)
    assert np.array_equal(np.argmax(M, axis=1), np.argmax(E, axis=1))


def test_calibrate_ties_prefer_smaller_index():
    keep = O.calibrate_row(np.array([1.0, 2.0, 2.0, 2.0]), 0.5)   # total 7, need 3.5
    assert keep.tolist() == [0, 1, 1, 0]


def test_calibrate_monotone_in_eps():
    rng = np.random.default_rng(4)
    E = rng.lognormal(0, 1, (15, 40))
    prev = np.zeros_like(E, dtype=np.uint8)
    for eps in (0.1, 0.3, 0.5, 0.7, 0.9, 0.99):
        M = O.calibrate_mask(E, eps)
        assert np.all(M >= prev)
        prev = M


def test_calibrate_brute_force_minimal_subset():
    rng = np.random.default_rng(5)
    for trial in range(20):
        E = rng.random(6)
        eps = rng.uniform(0.05, 0.99)
        keep = O.calibrate_row(E, eps)
        need = eps * E.sum()
        sizes = [len(c) for r in range(1, 7) for c in itertools.combinations(range(6), r)
                 if sum(E[list(c)]) >= need]
        assert keep.sum() == min(sizes)
        assert E[keep == 1].sum() >= need * (1 - 1e-12)


def test_static_workload_sparsity():
    w = S.get_workload("static_wan720p")
    kept = [O.calibrate_mask(S.energy_matrix(w, h), w.eps).mean() for h in (0, 7, 21, 39)]
    # 68 % block sparsity of the calibrated-mask workload
    assert abs(np.mean(kept) - 0.32) < 0.01
    M = O.calibrate_mask(S.energy_matrix(w, 0), w.eps)
    assert np.all(M.sum(axis=1) >= 1)          # eps > 0 never empties a row
