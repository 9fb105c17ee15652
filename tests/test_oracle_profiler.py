"""Pins of the oracle's online profiler (CPU only)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth as S


def _exact_inputs(kind, F=4, Hs=4, Ws=4, B=8, L=64.0):
    """q = k = L * e_cluster, clusters = frames ("spatial") or positions
    ("temporal").  Same-cluster logits are L^2 * scale = 1024 above every
    cross-cluster logit, so cross-cluster weights are exactly 0 in float64:
    the mask that covers the whole cluster reproduces dense attention."""
    S_ = Hs * Ws
    N = F * S_
    D = S_
    i = np.arange(N)
    cl = i // S_ if kind == "spatial" else i % S_
    q = np.zeros((N, D))
    q[i, cl] = L
    q = torch.from_numpy(q).to(torch.bfloat16).double().numpy()     # stays exact in bf16
    v = np.random.default_rng(0).standard_normal((N, D))
    scale = 1.0 / np.sqrt(D)
    gap = L * L * scale
    assert gap >= 1000.0 and np.exp(-gap) == 0.0
    return q[None], q[None].copy(), v[None], F, Hs, Ws, B, scale


@pytest.mark.parametrize("kind,expect", [("spatial", 0), ("temporal", 1)])
def test_exact_mask_is_selected(kind, expect):
    q, k, v, F, Hs, Ws, B, scale = _exact_inputs(kind)
    N = q.shape[1]
    # spatial: +/-1 frame (misses frames 2 and 3 for a frame-0 query);
    # temporal: token-major band +/-1 block (a position's 4 copies share a block)
    cand = O.online_candidate_masks(F, Hs, Ws, N, B, 1)
    idx = np.random.default_rng(1).choice(N, 16, replace=False)
    choice, err = O.profile_heads(q, k, v, F, Hs, Ws, B, scale, idx, cand)
    assert choice[0] == expect
    assert err[0, expect] < 1e-20 and err[0, 1 - expect] > 1e-3


def test_identical_candidates_tie_to_spatial():
    w = S.get_workload("tiny")
    q, k, v, _ = S.gen_qkv(w, dtype="f32")
    M = O.spatial_block_mask(w.F, w.Hs, w.Ws, w.N, w.block)
    cand = np.stack([M, M])
    # same mask in both slots is only equal as a token mask when the layouts
    # agree, so use the all-ones mask
    cand[:] = 1
    choice, err = O.profile_heads(q[0].numpy(), k[0].numpy(), v[0].numpy(), w.F, w.Hs, w.Ws,
                                  w.block, w.scale, S.sample_query_idx(w), cand)
    assert np.all(err == 0) and np.all(choice == 0)


def test_decomposition_equals_direct_errors():
    w = S.get_workload("tiny")
    q, k, v, _ = S.gen_qkv(w, dtype="f32")
    args = (q[0].double().numpy(), k[0].double().numpy(), v[0].double().numpy(),
            w.F, w.Hs, w.Ws, w.block, w.scale, S.sample_query_idx(w),
            O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w))
    _, err = O.profile_heads(*args)
    err2 = O.profile_errors_decomposed(*args)
    assert np.allclose(err2, err, rtol=1e-6, atol=0)


@pytest.mark.parametrize("name,heads", [("tiny", None), ("cogvideox", [0, 1, 2, 3, 4, 5]),
                                        ("wan720p", None), ("hunyuan720p", None)])
def test_generator_heads_are_recovered(name, heads):
    """Generator self-check: every generated head is labelled with its class."""
    w = S.get_workload(name)
    cls_all = S.head_classes(w)
    if heads is None:
        sp = [h for h in range(w.H) if cls_all[h] == 0][:2]
        tp = [h for h in range(w.H) if cls_all[h] == 1][:2]
        heads = sp + tp
    q, k, v, cls = S.gen_qkv(w, heads=heads)
    cand = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    choice, err = O.profile_heads(q[0].float().numpy(), k[0].float().numpy(), v[0].float().numpy(),
                                  w.F, w.Hs, w.Ws, w.block, w.scale, S.sample_query_idx(w), cand)
    assert np.array_equal(choice, cls)
    ratio = np.where(cls == 0, err[:, 1] / err[:, 0], err[:, 0] / err[:, 1])
    assert np.all(ratio >= 10.0)
