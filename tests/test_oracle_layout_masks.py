"""Pins of the oracle's permutation, block masks and anchor rows (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle as O
import synth as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_permutation_hand_case():
    g = _gold("permutation_F2_Hs2_Ws2.json")
    p = O.token_major_index(g["F"], g["Hs"], g["Ws"], g["N"])
    assert p.tolist() == g["p"]


@pytest.mark.parametrize("F,Hs,Ws,text", [(4, 16, 16, 0), (13, 30, 45, 0), (3, 5, 7, 9)])
def test_permutation_bijection_inverse_runs(F, Hs, Ws, text):
    S_ = Hs * Ws
    N = F * S_ + text
    p = O.token_major_index(F, Hs, Ws, N)
    assert np.array_equal(np.sort(p), np.arange(N))
    assert np.array_equal(p[F * S_:], np.arange(F * S_, N))
    x = np.random.default_rng(0).standard_normal((2, N, 3))
    y = O.to_token_major(x, F, Hs, Ws)
    assert np.array_equal(O.to_frame_major(y, F, Hs, Ws), x)
    for s in (0, S_ // 2, S_ - 1):       # the F copies of a position are one contiguous run
        run = y[:, s * F:(s + 1) * F]
        assert np.array_equal(run, x[:, [f * S_ + s for f in range(F)]])


def test_worked_example_is_tiny_workload():
    g = _gold("worked_example_tokens.json")
    w = S.get_workload("tiny")
    assert (g["frame_px"] // g["patch_px"]) ** 2 * g["frames"] == g["tokens"] == w.N
    assert (w.F, w.Hs, w.Ws) == (g["frames"], g["frame_px"] // g["patch_px"], g["frame_px"] // g["patch_px"])


def test_sample_fraction_matches_pages():
    g = _gold("sample_fraction.json")
    for name, n in g["video_tokens"].items():
        w = S.get_workload(name)
        assert w.N_video == n and w.n_samples == g["n_samples"]
        frac = g["n_samples"] / n
        assert min(g["quoted_fractions"]) <= round(frac, 4) <= max(g["quoted_fractions"])


def test_tiny_masks_closed_form():
    w = S.get_workload("tiny")
    Ms = O.spatial_block_mask(w.F, w.Hs, w.Ws, w.N, w.block)
    Mt = O.temporal_block_mask(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    # 4 frames of 4 aligned blocks: frame pairs at distance <= 1 are 4 + 2*3 = 10,
    # each a 4x4 block of blocks
    assert Ms.sum() == 10 * 16
    frame = np.arange(16) // 4
    assert np.array_equal(Ms, (np.abs(frame[:, None] - frame[None, :]) <= 1).astype(np.uint8))
    assert Mt.sum() == 16 + 2 * 15


@pytest.mark.parametrize("name", ["cogvideox", "wan720p", "hunyuan720p"])
def test_temporal_band_closed_form_and_width(name):
    w = S.get_workload(name)
    n = w.n_blocks
    Mt = O.temporal_block_mask(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    band = n * (2 * w.band_w + 1) - w.band_w * (w.band_w + 1)
    if w.text == 0:
        assert Mt.sum() == band
    # the workload's width is the smallest reaching 30 % kept blocks
    assert Mt.mean() >= 0.30
    Mt1 = O.temporal_block_mask(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w - 1)
    assert Mt1.mean() < 0.30
    assert np.array_equal(Mt, Mt.T) and np.all(np.diag(Mt) == 1)


def test_spatial_mask_brute_force_unaligned_frames():
    """CogVideoX shape: 10.55 blocks per frame.  Token-level check: a block pair
    is kept iff some video token pair is at most one frame apart."""
    w = S.get_workload("cogvideox")
    Ms = O.spatial_block_mask(w.F, w.Hs, w.Ws, w.N, w.block)
    f = np.arange(w.N) // w.S
    n = w.n_blocks
    pad = n * w.block - w.N
    fp = np.concatenate([f, np.full(pad, -100)])        # padding never pairs
    blk = fp.reshape(n, w.block)
    ref = np.zeros((n, n), bool)
    for r in range(n):
        d = np.abs(blk[r][:, None, None] - blk[None, :, :])   # [128, n, 128]
        ref[r] = (d <= 1).any(axis=(0, 2))
    assert np.array_equal(Ms.astype(bool), ref)
    assert Ms.sum() == 4384


def test_online_mask_kept_counts():
    # regression values of the kept-block counts (not printed on the pages)
    expect = {"wan720p": (49231, 105739), "hunyuan720p": (83819, 260699)}
    for name, (ks, kt) in expect.items():
        w = S.get_workload(name)
        M = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
        assert (int(M[0].sum()), int(M[1].sum())) == (ks, kt)
        assert np.array_equal(M[0], M[0].T) and np.all(np.diag(M[0]) == 1)


def test_text_rule_hunyuan():
    w = S.get_workload("hunyuan720p")
    M = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    assert w.n_blocks == 931 and w.N_video % w.block == 16   # block 928 mixes video and text
    for m in range(2):
        assert np.all(M[m, 928:] == 1) and np.all(M[m, :, 928:] == 1)
    assert M[0, 0, 927] == 0


def test_anchor_rows_and_saving():
    g = _gold("anchor_saving.json")
    a = O.anchor_rows(g["H"], g["k"])
    assert sorted(set(a.tolist())) == [4, 13, 22, 31, 40]
    assert 1 - len(set(a.tolist())) / g["H"] == pytest.approx(g["saving"], abs=1e-15)
    # every row maps to the anchor of its own band; k = Hs is the identity
    assert np.array_equal(O.anchor_rows(7, 7), np.arange(7))
    w = S.get_workload("static_wan720p")
    blocks = O.anchor_query_blocks(w.F, w.Hs, w.Ws, w.N, w.block, w.k_anchors)
    assert blocks.sum() == 158


def test_row_broadcast():
    F, Hs, Ws, k = 3, 9, 4, 3
    N = F * Hs * Ws + 5
    o = np.random.default_rng(1).standard_normal((N, 6))
    b = O.row_broadcast(o, F, Hs, Ws, k)
    a = O.anchor_rows(Hs, k)
    for f in range(F):
        for y in range(Hs):
            row = slice(f * Hs * Ws + y * Ws, f * Hs * Ws + (y + 1) * Ws)
            src = slice(f * Hs * Ws + a[y] * Ws, f * Hs * Ws + (a[y] + 1) * Ws)
            assert np.array_equal(b[row], o[src])
            if y == a[y]:
                assert np.array_equal(b[row], o[row])
    assert np.array_equal(b[F * Hs * Ws:], o[F * Hs * Ws:])
    assert np.array_equal(O.row_broadcast(o, F, Hs, Ws, Hs), o)


# ---- row-repetitive head test: mean cosine of the rows' attention patterns

def test_row_similarity_uniform_attention_is_one():
    # q = 0: every query spreads its weight evenly, so all rows share one pattern
    F, Hs, Ws = 2, 4, 8
    N = F * Hs * Ws + 5                                   # a text tail as well
    rng = np.random.default_rng(31)
    A = O.row_patterns(np.zeros((N, 16)), rng.standard_normal((N, 16)), 1.0, F, Hs, Ws)
    np.testing.assert_allclose(A, Ws / N, rtol=1e-12)
    assert abs(O.row_similarity(np.zeros((N, 16)), rng.standard_normal((N, 16)), 1.0, F, Hs, Ws) - 1) < 1e-12
    assert O.is_row_repetitive(1.0) and not O.is_row_repetitive(0.87)


def test_row_similarity_rows_attending_their_own_row_is_zero():
    # keys of each latent row point along their own orthonormal direction and
    # the queries of a row along their row's direction, with a large scale:
    # row patterns sit on disjoint key sets, every cosine is 0
    F, Hs, Ws, D = 2, 3, 4, 8
    N = F * Hs * Ws
    rng = np.random.default_rng(32)
    U = np.linalg.qr(rng.standard_normal((D, D)))[0][:, :F * Hs].T
    rows = np.repeat(np.arange(F * Hs), Ws)
    assert O.row_similarity(U[rows] * 60.0, U[rows], 1.0, F, Hs, Ws) < 1e-12


def test_row_similarity_two_groups_closed_form():
    # rows y < Hs/2 attend (evenly) to key set A, the others to key set B,
    # disjoint: a pair in one group has cosine 1, a mixed pair 0, so the mean
    # is 2 C(Hs/2, 2) / C(Hs, 2) = 1/3 for Hs = 4
    F, Hs, Ws, D = 3, 4, 5, 8
    N = F * Hs * Ws
    e = np.eye(D)
    y = (np.arange(N) // Ws) % Hs
    q = np.where((y < Hs // 2)[:, None], e[0], e[1]) * 50.0
    k = np.where((y < Hs // 2)[:, None], e[0], e[1])
    assert abs(O.row_similarity(q, k, 1.0, F, Hs, Ws) - 1.0 / 3.0) < 1e-12
