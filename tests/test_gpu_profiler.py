"""GPU parity of the online head profiler.

Head choice must equal the oracle's on every compared head (bit-exact); the
reported errors must match the float64 oracle within PROFILE_ERR_REL.  The
full-size workloads (every head) are in test_gpu_full_size.py.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_svg_amd as svg
import oracle as O
import synth as S
from parity_utils import banner, PROFILE_ERR_REL

pytestmark = pytest.mark.gpu
DEV = "cuda"
ERR_REL = PROFILE_ERR_REL


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


@pytest.mark.parametrize("name,heads", [("tiny", None), ("cogvideox", None)])
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
    print(f"[profile] {name}: worst relative error deviation {rel.max():.2e}")
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
    rel = np.abs(err - ref_e) / ref_e
    print(f"[profile] 37 samples: worst relative error deviation {rel.max():.2e}")
    assert np.all(rel < ERR_REL)


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


def _blend(w, alpha):
    """q, k of a spatial generator head and a temporal one mixed with weight
    alpha (alpha = 1: the spatial head), v of the spatial head; bf16."""
    qs, ks, vs = S.gen_head_qkv(w, 0, 0)                 # class 0: spatial
    qt, kt, _ = S.gen_head_qkv(w, 1, 1)                  # class 1: temporal
    tb = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    return tb(alpha * qs + (1 - alpha) * qt), tb(alpha * ks + (1 - alpha) * kt), tb(vs)


def _near_tie_inputs(w, idx, cand, target):
    """Blend weight whose oracle error ratio e_spatial / e_temporal is about
    `target` (bisection on the oracle alone; the ratio falls as alpha grows)."""
    def ratio(alpha):
        q, k, v = _blend(w, alpha)
        _, e = O.profile_heads(q[None].float().numpy(), k[None].float().numpy(), v[None].float().numpy(),
                               w.F, w.Hs, w.Ws, w.block, w.scale, idx, cand)
        return e[0, 0] / e[0, 1]
    lo, hi = 0.0, 1.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if ratio(mid) > target:
            lo = mid
        else:
            hi = mid
    return _blend(w, 0.5 * (lo + hi))


def test_near_tie_heads_choose_as_oracle():
    """Heads whose two candidate errors are 1 % and 0.5 % apart, either way:
    the choice is the oracle's and each error is within PROFILE_ERR_REL."""
    banner("profile near tie")
    w = S.get_workload("cogvideox", H=4, F=4, Hs=12, Ws=16, n_spatial=1, band_w=1, sigma=0.3, seed=5)
    idx = S.sample_query_idx(w, 0)
    cand = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    targets = [1.01, 1 / 1.01, 1.005, 1 / 1.005]
    heads = [_near_tie_inputs(w, idx, cand, t) for t in targets]
    q, k, v = (torch.stack([h[i] for h in heads])[None] for i in range(3))
    ref_c, ref_e = O.profile_heads(q[0].float().numpy(), k[0].float().numpy(), v[0].float().numpy(),
                                   w.F, w.Hs, w.Ws, w.block, w.scale, idx, cand)
    ratio = ref_e[:, 0] / ref_e[:, 1]
    for t, r in zip(targets, ratio):                 # the construction reached its targets
        assert abs(np.log(r / t)) < 2e-3, (t, r)
    choice, err = _gpu_profile(w, q, k, v, idx, cand_np=cand)
    rel = np.abs(err - ref_e) / ref_e
    print(f"[near tie] oracle ratios {np.round(ratio, 5).tolist()}, GPU ratios "
          f"{np.round(err[:, 0] / err[:, 1], 5).tolist()}, worst relative error deviation {rel.max():.2e}")
    assert np.array_equal(ref_c, [1, 0, 1, 0])
    assert np.array_equal(choice, ref_c)
    assert np.all(rel < ERR_REL)


@pytest.mark.parametrize("seed", range(10))
def test_random_shapes_match_oracle(seed):
    """Seeded random shapes (2-11 frames, 4-19 rows, frames of a multiple of 8
    tokens two times in three and of an odd size otherwise, text tails, both block sizes and head dims,
    temporal bands of 1-3 blocks, several key chunks).  Each error within
    PROFILE_ERR_REL of the oracle's, relative to the oracle's value or, for a
    mask that is nearly exact for the head, to 1e-6 of the head's larger
    error; the oracle's choice wherever its two errors are more than 3 %
    apart (closer ties are the near-tie test's); both errors 0 (masks that
    keep every block) give 0 on the GPU and the spatial mask."""
    rng = np.random.default_rng(5200 + seed)
    block = (64, 128)[seed % 2]
    D = (64, 128)[(seed // 2) % 2]
    F, Hs = int(rng.integers(2, 12)), int(rng.integers(4, 20))
    if seed % 3:
        Ws = 8 * int(rng.integers(1, 5))                  # frames of a multiple of 8 tokens
    else:
        Hs, Ws = Hs | 1, 2 * int(rng.integers(1, 15)) + 1   # odd frame sizes
    text = int(rng.integers(1, 150)) if rng.random() < 0.5 else 0
    w = S.get_workload("cogvideox", H=2, D=D, F=F, Hs=Hs, Ws=Ws, text=text, block=block,
                       band_w=int(rng.integers(1, 4)), sigma=float(rng.uniform(0.1, 0.4)), n_spatial=1,
                       seed=5300 + seed)
    banner("profile random shape", seed, f"D{D} block {block} {F}x{Hs}x{Ws} + {text} text")
    q, k, v, cls = S.gen_qkv(w, dtype="bf16")
    idx = S.sample_query_idx(w, seed)
    choice, err = _gpu_profile(w, q, k, v, idx)
    cand = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    ref_c, ref_e = O.profile_heads(q[0].float().numpy(), k[0].float().numpy(), v[0].float().numpy(),
                                   w.F, w.Hs, w.Ws, w.block, w.scale, idx, cand)
    top = ref_e.max(axis=1, keepdims=True)
    zero = top[:, 0] == 0
    assert np.all(err[zero] == 0) and np.all(choice[zero] == 0), (err, choice)
    den = np.maximum(ref_e, 1e-6 * top)[~zero]
    rel = np.abs(err[~zero] - ref_e[~zero]) / den
    print(f"[profile random {seed}] oracle ratios {ref_e[:, 0] / np.maximum(ref_e[:, 1], 1e-300)}, "
          f"worst relative error deviation {rel.max() if rel.size else 0.0:.2e}")
    assert np.all(rel < ERR_REL), (rel.max(), err, ref_e)
    with np.errstate(divide="ignore", invalid="ignore"):
        clear = np.abs(np.log(ref_e[:, 0] / ref_e[:, 1])) > 0.03
    assert np.array_equal(choice[clear], ref_c[clear]), (choice, ref_c, ref_e)
