"""Pins of the oracle's dense and block-masked attention (CPU only)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth as S


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa(q, k, v, mask=None, scale=None):
    """torch's fp64 CPU scaled_dot_product_attention (a library routine)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    am = None if mask is None else torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=am, scale=scale)
    return o[0, 0].numpy()


def test_dense_matches_library_sdpa():
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 37, 24), _rand(rng, 53, 24), _rand(rng, 53, 24)
    o, _ = O.dense_attention(q, k, v, 24 ** -0.5)
    assert np.max(np.abs(o - _sdpa(q, k, v))) < 1e-12


def test_dense_matches_naive_loops():
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 5, 3), _rand(rng, 7, 3), _rand(rng, 7, 3)
    scale = 0.7
    o, lse = O.dense_attention(q, k, v, scale)
    for i in range(5):
        s = [scale * sum(q[i, d] * k[j, d] for d in range(3)) for j in range(7)]
        w = [np.exp(x) for x in s]
        z = sum(w)
        for d in range(3):
            assert abs(o[i, d] - sum(w[j] * v[j, d] for j in range(7)) / z) < 1e-12
        assert abs(lse[i] - np.log(z)) < 1e-12


def test_rows_sum_to_one_and_lse():
    rng = np.random.default_rng(3)
    q, k = _rand(rng, 20, 16) * 3, _rand(rng, 30, 16) * 3
    P, lse = O.dense_attention(q, k, np.eye(30), 0.25)   # v = I gives the weights
    assert np.max(np.abs(P.sum(axis=1) - 1.0)) < 1e-12
    assert np.all(P >= 0)
    ref = torch.logsumexp(torch.from_numpy(q @ k.T * 0.25), dim=1).numpy()
    assert np.max(np.abs(lse - ref)) < 1e-12


def test_constant_v_gives_constant_output():
    rng = np.random.default_rng(4)
    q, k = _rand(rng, 9, 8), _rand(rng, 11, 8)
    v = np.tile(rng.standard_normal(8), (11, 1))
    o, _ = O.dense_attention(q, k, v, 1.0)
    assert np.max(np.abs(o - v[0])) < 1e-12


def test_single_admitted_key_is_exact():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 6, 4), _rand(rng, 6, 4), _rand(rng, 6, 4)
    M = np.zeros((6, 6), np.uint8)
    cols = [3, 0, 5, 5, 1, 2]
    M[np.arange(6), cols] = 1
    o, lse = O.block_masked_attention(q, k, v, M, 1, 0.5)
    assert np.array_equal(o, v[cols])
    assert np.allclose(lse, 0.5 * np.sum(q * k[cols], axis=1), atol=1e-15)


def test_all_ones_mask_equals_dense():
    rng = np.random.default_rng(6)
    N, B = 200, 32
    q, k, v = _rand(rng, N, 16), _rand(rng, N, 16), _rand(rng, N, 16)
    nb = -(-N // B)
    o, lse = O.block_masked_attention(q, k, v, np.ones((nb, nb), np.uint8), B, 0.25)
    od, lsed = O.dense_attention(q, k, v, 0.25)
    assert np.max(np.abs(o - od)) < 1e-12 and np.max(np.abs(lse - lsed)) < 1e-12


def test_block_diagonal_is_independent_attention():
    rng = np.random.default_rng(7)
    N, B = 100, 16
    q, k, v = _rand(rng, N, 8), _rand(rng, N, 8), _rand(rng, N, 8)
    nb = -(-N // B)
    o, _ = O.block_masked_attention(q, k, v, np.eye(nb, dtype=np.uint8), B, 0.3)
    for b in range(nb):
        sl = slice(b * B, min(N, (b + 1) * B))
        assert np.max(np.abs(o[sl] - _sdpa(q[sl], k[sl], v[sl], scale=0.3))) < 1e-12


def test_brute_force_token_mask_on_tiny():
    """Block mask expanded to a token-level -inf mask in one 1024x1024 softmax."""
    w = S.get_workload("tiny")
    rng = np.random.default_rng(8)
    q, k, v = (_rand(rng, w.N, w.D) for _ in range(3))
    M = O.spatial_block_mask(w.F, w.Hs, w.Ws, w.N, w.block)
    blk = np.arange(w.N) // w.block
    tok = M[blk[:, None], blk[None, :]] != 0
    o, _ = O.block_masked_attention(q, k, v, M, w.block, w.scale)
    assert np.max(np.abs(o - _sdpa(q, k, v, mask=tok, scale=w.scale))) < 1e-12


def test_permutation_equivariance():
    """Token-major attention then inverse permute == frame-major attention under
    the token mask pulled back through the permutation."""
    w = S.get_workload("tiny")
    rng = np.random.default_rng(9)
    q, k, v = (_rand(rng, w.N, w.D) for _ in range(3))
    M = O.temporal_block_mask(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    o, _ = O.head_attention(q, k, v, M, 1, w.F, w.Hs, w.Ws, w.block, w.scale)
    pb = O.token_major_index(w.F, w.Hs, w.Ws, w.N) // w.block
    tok = M[pb[:, None], pb[None, :]] != 0
    assert np.max(np.abs(o - _sdpa(q, k, v, mask=tok, scale=w.scale))) < 1e-12


def test_empty_row_gives_zero_and_neg_inf():
    rng = np.random.default_rng(10)
    q, k, v = (_rand(rng, 64, 8) for _ in range(3))
    M = np.ones((4, 4), np.uint8)
    M[2] = 0
    o, lse = O.block_masked_attention(q, k, v, M, 16, 0.3)
    assert np.all(o[32:48] == 0) and np.all(np.isneginf(lse[32:48]))
    assert np.all(np.isfinite(lse[:32]))


def test_partial_last_block_and_subset():
    rng = np.random.default_rng(11)
    N, B = 150, 64                      # last block holds 22 tokens
    q, k, v = (_rand(rng, N, 8) for _ in range(3))
    M = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 1]], np.uint8)
    o, _ = O.block_masked_attention(q, k, v, M, B, 0.3, qblocks=[2])
    assert np.all(np.isnan(o[:128]))
    assert np.max(np.abs(o[128:] - _sdpa(q[128:], k, v, scale=0.3))) < 1e-12


def test_algorithmic_flops():
    N, B, D = 150, 64, 8
    assert O.kept_pairs(np.ones((3, 3), np.uint8), N, B) == N * N
    M = np.array([[1, 0, 0], [0, 0, 0], [0, 0, 1]], np.uint8)
    assert O.kept_pairs(M, N, B) == 64 * 64 + 22 * 22
    assert O.algorithmic_flops([M, M], N, B, D) == 2 * 4 * D * (64 * 64 + 22 * 22)
