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


# ---- block energy, eps(t) schedule and the cross-prompt merge ([CalibAtt] section 3.1)

def test_block_energy_rows_sum_to_query_counts():
    # every query's softmax weights sum to 1, so row r of E sums to |r|;
    # N = 300 with 64-blocks leaves a ragged last block of 44 queries
    rng = np.random.default_rng(11)
    q = rng.standard_normal((300, 32))
    k = rng.standard_normal((300, 32))
    E = O.block_energy(q, k, 0.3, 64)
    assert E.shape == (5, 5)
    np.testing.assert_allclose(E.sum(axis=1), [64, 64, 64, 64, 44], rtol=0, atol=1e-9)
    assert (E > 0).all()


def test_block_energy_uniform_attention():
    # q = 0: every weight is 1/N, so E[r, c] = |r| |c| / N
    N, B = 200, 64
    rng = np.random.default_rng(12)
    E = O.block_energy(np.zeros((N, 16)), rng.standard_normal((N, 16)), 1.0, B)
    sizes = np.array([64, 64, 64, 8], dtype=np.float64)
    np.testing.assert_allclose(E, np.outer(sizes, sizes) / N, rtol=1e-12)


def test_block_energy_one_hot_attention_is_not_transposed():
    # keys are orthonormal directions and query i points along key f(i), with a
    # large scale: query i puts all its weight on key f(i), so E[r, c] counts
    # the queries of block r whose partner lies in block c.  f is chosen so
    # that this count matrix is not symmetric.
    N, D, B = 48, 64, 16
    rng = np.random.default_rng(13)
    basis = np.linalg.qr(rng.standard_normal((D, D)))[0][:, :N].T   # N orthonormal rows
    f = np.array([(3 * i + 17) % N if i < 16 else (i + 16) % N for i in range(N)])
    E = O.block_energy(basis[f] * 40.0, basis, 1.0, B)
    want = np.zeros((3, 3))
    for i in range(N):
        want[i // B, f[i] // B] += 1
    assert not np.array_equal(want, want.T)
    np.testing.assert_allclose(E, want, atol=1e-9)


def test_block_energy_ignores_key_order_within_a_block():
    rng = np.random.default_rng(14)
    q = rng.standard_normal((128, 16))
    k = rng.standard_normal((128, 16))
    perm = np.concatenate([rng.permutation(32) + 32 * b for b in range(4)])
    np.testing.assert_allclose(O.block_energy(q, k[perm], 0.5, 32), O.block_energy(q, k, 0.5, 32),
                               rtol=1e-12)


def test_eps_schedule_ends_midpoint_and_decay():
    assert O.eps_schedule(0, 50) == 0.99
    assert abs(O.eps_schedule(49, 50) - 0.84) < 1e-15
    assert abs(O.eps_schedule(10, 21) - np.sqrt(0.99 * 0.84)) < 1e-15   # geometric midpoint
    v = [O.eps_schedule(t, 50) for t in range(50)]
    assert all(a > b for a, b in zip(v, v[1:]))
    assert O.eps_schedule(0, 1) == 0.99


def test_aggregate_masks_frequency_rule():
    rng = np.random.default_rng(15)
    M = (rng.random((4, 2, 6, 6)) < 0.5).astype(np.uint8)
    np.testing.assert_array_equal(O.aggregate_masks(M[:1], 0.5), M[0])
    np.testing.assert_array_equal(O.aggregate_masks(M, 1e-9), M.max(axis=0))     # union
    np.testing.assert_array_equal(O.aggregate_masks(M, 1.0), M.min(axis=0))      # intersection
    want = np.zeros_like(M[0])
    for idx in itertools.product(*(range(n) for n in M.shape[1:])):
        kept = sum(int(M[(p,) + idx]) for p in range(4))
        want[idx] = 1 if 2 * kept >= 4 else 0                                    # rho = 0.5
    np.testing.assert_array_equal(O.aggregate_masks(M, 0.5), want)
