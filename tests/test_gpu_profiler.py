"""GPU parity of the online head profiler.

Head choice must equal the oracle's on every compared head (bit-exact); the
reported errors must match the float64 oracle within a relative 5e-2 (the GPU
sums bf16-rounded softmax weights in fp32).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_svg_amd as svg
import oracle as O
import synth as S
from parity_utils import banner

pytestmark = pytest.mark.gpu
DEV = "cuda"
ERR_REL = 5e-2


def shape_of(w, H=None):
    return svg.Shape(w.B, H or w.H, w.N, w.D, w.F, w.Hs, w.Ws, w.block)


def _gpu_profile(w, q, k, v, idx, cand_np=None, band_w=None):
    s = shape_of(w, q.shape[1])
    if cand_np is None:
        dense = svg.svg_build_masks(s, w.band_w if band_w is None else band_w)
    else:
        dense = torch.from_numpy(np.ascontiguousarray(cand_np)).to(DEV)
    cand = svg.svg_encode_mask(dense)
    idx_d = torch.from_numpy(np.asarray(idx, np.int32)).to(DEV)
    choice, err = svg.svg_profile_heads(q.to(DEV), k.to(DEV), v.to(DEV), s, 1.0 / np.sqrt(w.D),
                                        idx_d, cand)
    torch.cuda.synchronize()
    return choice.cpu().numpy(), err.cpu().numpy()


@pytest.mark.parametrize("name,heads", [("tiny", None), ("cogvideox", None),
                                        ("wan720p", [0, 1, 2, 3, 17, 39]),
                                        ("hunyuan720p", [0, 5, 11, 23])])
def test_profile_matches_oracle(name, heads, workload_inputs):
    banner("profile", name)
    w, q, k, v, cls = workload_inputs(name, dtype="bf16")
    idx = S.sample_query_idx(w, 0)
    choice, err = _gpu_profile(w, q, k, v, idx)          # every head, as in the layer
    assert np.array_equal(choice, cls), "generator classes"
    cand = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    heads = list(range(w.H)) if heads is None else heads
    ref_c, ref_e = O.profile_heads(q[0, heads].float().numpy(), k[0, heads].float().numpy(),
                                   v[0, heads].float().numpy(), w.F, w.Hs, w.Ws, w.block, w.scale,
                                   idx, cand)
    assert np.array_equal(choice[heads], ref_c)
    rel = np.abs(err[heads] - ref_e) / np.maximum(ref_e, 1e-30)
    assert np.all(rel < ERR_REL), (rel.max(), err[heads], ref_e)


def test_profile_partial_sample_count(workload_inputs):
    banner("profile 37 samples")
    w, q, k, v, cls = workload_inputs("cogvideox", dtype="bf16")
    idx = S.sample_query_idx(w, 3)[:37]
    heads = [0, 1, 2, 3]
    choice, err = _gpu_profile(w, q[:, heads].contiguous(), k[:, heads].contiguous(),
                               v[:, heads].contiguous(), idx)
    cand = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    ref_c, ref_e = O.profile_heads(q[0, heads].float().numpy(), k[0, heads].float().numpy(),
                                   v[0, heads].float().numpy(), w.F, w.Hs, w.Ws, w.block, w.scale,
                                   idx, cand)
    assert np.array_equal(choice, ref_c)
    assert np.all(np.abs(err - ref_e) / ref_e < ERR_REL)


def _exact_inputs(kind, F=4, Hs=4, Ws=4, L=64.0):
    """q = k = L * e_cluster with clusters = frames or positions; cross-cluster
    weights underflow to 0, so the mask covering the cluster is exact."""
    S_ = Hs * Ws
    N = F * S_
    D = 64
    i = np.arange(N)
    cl = i // S_ if kind == "spatial" else i % S_
    qk = np.zeros((N, D))
    qk[i, cl] = L
    v = np.random.default_rng(0).standard_normal((N, D))
    t = lambda a: torch.from_numpy(a[None, None].astype(np.float32)).to(torch.bfloat16)
    return t(qk), t(qk), t(v), N


@pytest.mark.parametrize("kind,expect", [("spatial", 0), ("temporal", 1)])
def test_exact_mask_inputs_select_exact_mask(kind, expect):
    """4 frames of 8x8 positions, block 64 = one frame.  Spatial +/-1 frame
    misses a position's copy two frames away; the temporal band of +/-1
    token-major block holds all 4 copies of a position but not a whole frame."""
    banner("profile exact", kind)
    w = S.get_workload("tiny", H=1, D=64, F=4, Hs=8, Ws=8, block=64)
    q, k, v, N = _exact_inputs(kind, F=4, Hs=8, Ws=8, L=128.0)   # logit gap 2048
    idx = np.random.default_rng(1).choice(N, 16, replace=False).astype(np.int32)
    cand = O.online_candidate_masks(w.F, w.Hs, w.Ws, N, w.block, 1)
    choice, err = _gpu_profile(w, q, k, v, idx, cand_np=cand)
    ref_c, ref_e = O.profile_heads(q[0].float().numpy(), k[0].float().numpy(), v[0].float().numpy(),
                                   w.F, w.Hs, w.Ws, w.block, w.scale, idx, cand)
    assert ref_c[0] == expect and choice[0] == expect
    assert err[0, expect] < 1e-6 * err[0, 1 - expect]


def test_identical_candidates_tie_to_spatial(workload_inputs):
    banner("profile tie")
    w, q32, k32, v32, _ = workload_inputs("tiny", dtype="f32")
    q, k, v = (t.to(torch.bfloat16) for t in (q32, k32, v32))
    cand = np.ones((2, w.n_blocks, w.n_blocks), np.uint8)
    choice, err = _gpu_profile(w, q, k, v, S.sample_query_idx(w), cand_np=cand)
    assert np.all(err == 0) and np.all(choice == 0)


def test_profile_is_deterministic(workload_inputs):
    banner("profile determinism")
    w, q, k, v, _ = workload_inputs("cogvideox", dtype="bf16")
    idx = S.sample_query_idx(w, 1)
    c1, e1 = _gpu_profile(w, q, k, v, idx)
    c2, e2 = _gpu_profile(w, q, k, v, idx)
    assert np.array_equal(c1, c2) and np.array_equal(e1.view(np.uint32), e2.view(np.uint32))
