"""GPU parity of the offline calibration steps ([CalibAtt] section 3.1): block
attention energies against the float64 oracle, the merge of candidate masks
and the eps(t) schedule bit for bit, and the whole chain (energies of several
prompts -> threshold masks -> merge) against the oracle's rules."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_svg_amd as svg
import oracle as O
import synth as S
from parity_utils import banner

pytestmark = pytest.mark.gpu
DEV = "cuda"
U = 2.0 ** -24   # fp32 unit roundoff


def energy_bound(q, k, scale, B, rows=None):
    """Oracle energies of the query blocks `rows` and a per-entry bound on the
    GPU's error, from its fp32 arithmetic: each score carries at most
    (D + 2) u |q_i| |k_j| of accumulation error, the log-sum-exp the largest
    such score error plus the rounding of an N-term sum and of log2, each
    weight a further fma, exp2 and scaling rounding, and each block sum the
    rounding of a 64-term lane sum and a 6 + 4 step tree."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    N, D = q.shape
    nB = -(-N // B)
    rows = range(nB) if rows is None else rows
    c2 = scale / math.log(2.0)
    kn = np.linalg.norm(k, axis=1)
    E = np.zeros((len(rows), nB))
    bound = np.zeros((len(rows), nB))
    for a, r in enumerate(rows):
        qi = q[r * B:(r + 1) * B]
        s = (qi @ k.T) * scale
        lse = np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1)
        p = np.exp(s - lse[:, None])
        ds = c2 * (D + 2) * U * np.outer(np.linalg.norm(qi, axis=1), kn)   # log2 units
        dlse = ds.max(1) + (N / 64 + 64) * U / math.log(2.0) + 4 * U
        t = np.abs(s * (1 / math.log(2.0))) + np.abs(lse / math.log(2.0))[:, None]
        rel = math.log(2.0) * (ds + dlse[:, None] + 2 * U * t) + 4 * U
        for c in range(nB):
            blk = slice(c * B, (c + 1) * B)
            E[a, c] = p[:, blk].sum()
            bound[a, c] = (p[:, blk] * rel[:, blk]).sum() + 80 * U * E[a, c] + 1e-12
    return E, bound


def _qk(B_, H, N, D, seed, spread=1.0):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(B_, H, N, D, generator=g) * spread).to(torch.bfloat16)
    k = (torch.randn(B_, H, N, D, generator=g) * spread).to(torch.bfloat16)
    return q, k


@pytest.mark.parametrize("D,block,N", [(64, 64, 1024), (128, 128, 1000), (64, 128, 777), (128, 64, 600),
                                         (128, 128, 128), (64, 128, 130), (128, 128, 1)])
def test_block_energy_matches_oracle(D, block, N):
    banner(f"energy D={D} block={block} N={N}")
    q, k = _qk(1, 2, N, D, seed=D + block + N, spread=1.3)
    s = svg.Shape(1, 2, N, D, 1, 1, N, block)
    scale = 1.0 / math.sqrt(D)
    E = svg.svg_block_energy(q.to(DEV), k.to(DEV), s, scale).cpu().numpy()
    torch.cuda.synchronize()
    nB = -(-N // block)
    sizes = np.array([min(block, N - r * block) for r in range(nB)], np.float64)
    for h in range(2):
        ref, bound = energy_bound(q[0, h].float().numpy(), k[0, h].float().numpy(), scale, block)
        err = np.abs(E[h] - ref)
        assert (err <= bound).all(), f"head {h}: max err {err.max():.3e}, worst err/bound {(err / bound).max():.3f}"
        np.testing.assert_allclose(E[h].sum(1), sizes, rtol=1e-4)


def test_block_energy_is_deterministic():
    banner("energy determinism")
    q, k = _qk(1, 3, 900, 128, seed=5)
    s = svg.Shape(1, 3, 900, 128, 1, 1, 900, 128)
    a = svg.svg_block_energy(q.to(DEV), k.to(DEV), s, 0.09)
    b = svg.svg_block_energy(q.to(DEV), k.to(DEV), s, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_block_energy_full_wan_shape_sampled_rows(workload_inputs):
    # two heads of the Wan 720p layer (one spatial, one temporal), 75,600 tokens:
    # every row sums to its query count, sampled rows match the oracle
    banner("energy wan720p sampled")
    w, q, k, v, cls = workload_inputs("wan720p")
    heads = [int(np.nonzero(cls == 0)[0][0]), int(np.nonzero(cls == 1)[0][0])]
    qs = q[:, heads].contiguous()
    ks = k[:, heads].contiguous()
    s = svg.Shape(1, 2, w.N, w.D, w.F, w.Hs, w.Ws, w.block)
    E = svg.svg_block_energy(qs.to(DEV), ks.to(DEV), s, w.scale).cpu().numpy()
    torch.cuda.synchronize()
    nB = w.n_blocks
    sizes = np.array([min(w.block, w.N - r * w.block) for r in range(nB)], np.float64)
    for a in range(2):
        qa, ka = qs[0, a].double().numpy(), ks[0, a].double().numpy()
        rows = [0, 1, nB // 2, nB - 1]
        ref, bound = energy_bound(qa, ka, w.scale, w.block, rows)
        err = np.abs(E[a][rows] - ref)
        assert (err <= bound).all(), f"head {heads[a]}: worst err/bound {(err / bound).max():.3f}"
        # every row sums to its query count, within the same arithmetic bound
        # taken with the largest norms (|s| <= |q| |k| scale bounds every term)
        c2 = w.scale / math.log(2.0)
        qk = np.linalg.norm(qa, axis=1).max() * np.linalg.norm(ka, axis=1).max()
        ds = c2 * (w.D + 2) * U * qk
        t_max = 2 * qk * c2 + math.log2(w.N)
        rel = math.log(2.0) * (2 * ds + (w.N / 64 + 64) * U / math.log(2.0) + 4 * U + 2 * U * t_max) + 84 * U
        np.testing.assert_allclose(E[a].sum(1), sizes, rtol=rel, atol=0)


def test_aggregate_masks_bit_exact():
    banner("aggregate masks")
    rng = np.random.default_rng(21)
    for n_sets, shape in [(5, (2, 37, 41)), (1, (3, 8, 8)), (4, (40, 20, 20))]:
        M = (rng.random((n_sets,) + shape) < 0.45).astype(np.uint8)
        Mg = torch.from_numpy(M).to(DEV)
        for rho in (0.5, 0.2, 0.6, 1.0):
            got = svg.svg_aggregate_masks(Mg, rho).cpu().numpy()
            np.testing.assert_array_equal(got, O.aggregate_masks(M, rho), err_msg=f"{n_sets} sets rho {rho}")


def test_eps_schedule_matches_oracle():
    for T in (1, 2, 7, 50):
        for t in range(T):
            a = svg.svg_eps_schedule(t, T)
            b = O.eps_schedule(t, T)
            assert abs(a - b) <= 2e-16 * b, (t, T, a, b)
    assert svg.svg_eps_schedule(0, 50) == 0.99


def test_calibration_chain_from_gpu_energies():
    # three prompts (seeds) of a small two-head layer: energies on the GPU,
    # per-prompt threshold masks at step t's eps, then the rho = 0.5 merge;
    # every decision is re-taken by the oracle's rules on the same energies
    banner("calibration chain")
    w = S.get_workload("tiny")
    s = svg.Shape(1, w.H, w.N, w.D, w.F, w.Hs, w.Ws, w.block)
    t, T = 12, 40
    eps = svg.svg_eps_schedule(t, T)
    energies, cands = [], []
    for seed in range(3):
        q, k, _, _ = S.gen_qkv(dataclasses.replace(w, seed=w.seed + 100 * seed), dtype="bf16")
        E = svg.svg_block_energy(q.to(DEV), k.to(DEV), s, w.scale)
        cands.append(svg.svg_calibrate_masks(E, eps))
        energies.append(E.cpu().numpy())
        ref, bound = energy_bound(q[0, 0].float().numpy(), k[0, 0].float().numpy(), w.scale, w.block)
        assert (np.abs(energies[-1][0] - ref) <= bound).all()
    merged = svg.svg_aggregate_masks(torch.stack(cands), 0.5).cpu().numpy()
    torch.cuda.synchronize()
    want_c = np.stack([np.stack([O.calibrate_mask(E[h], eps) for h in range(w.H)]) for E in energies])
    np.testing.assert_array_equal(torch.stack(cands).cpu().numpy(), want_c)
    np.testing.assert_array_equal(merged, O.aggregate_masks(want_c, 0.5))
    # a merged mask keeps every row's most energetic block of the majority of prompts
    assert merged.sum() > 0


# ---- row-repetitive head test ([CalibAtt] section 3.2) ------------------------

def _pattern_bound(q, k, scale, Ws, rows):
    """Oracle row patterns of `rows` and the largest relative error an entry may
    carry: each weight's fp32 error (as in energy_bound) plus a 128-term sum."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    N, D = q.shape
    c2 = scale / math.log(2.0)
    kn = np.linalg.norm(k, axis=1)
    A = np.zeros((len(rows), N))
    worst = 0.0
    for a, r in enumerate(rows):
        qi = q[r * Ws:(r + 1) * Ws]
        s = (qi @ k.T) * scale
        lse = np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1)
        p = np.exp(s - lse[:, None])
        ds = c2 * (D + 2) * U * np.outer(np.linalg.norm(qi, axis=1), kn)
        dlse = ds.max(1) + (N / 64 + 64) * U / math.log(2.0) + 4 * U
        t = np.abs(s / math.log(2.0)) + np.abs(lse / math.log(2.0))[:, None]
        rel = math.log(2.0) * (ds + dlse[:, None] + 2 * U * t) + 4 * U
        A[a] = p.sum(0)
        worst = max(worst, float(((p * rel).sum(0) / A[a]).max()) + 128 * U)
    return A, worst


@pytest.mark.parametrize("F,Hs,Ws,text,D", [(3, 6, 20, 10, 64), (2, 4, 100, 0, 128), (4, 16, 16, 0, 64),
                                            (3, 5, 33, 7, 128), (1, 3, 128, 50, 64), (2, 20, 4, 3, 64),
                                            (2, 37, 3, 0, 128), (2, 50, 3, 5, 128), (1, 64, 2, 9, 64)])
def test_row_similarity_matches_oracle(F, Hs, Ws, text, D):
    banner(f"row similarity F={F} Hs={Hs} Ws={Ws} D={D}")
    N = F * Hs * Ws + text
    q, k = _qk(1, 2, N, D, seed=F * 100 + Hs + Ws, spread=1.2)
    s = svg.Shape(1, 2, N, D, F, Hs, Ws, 64)
    scale = 1.0 / math.sqrt(D)
    ws = torch.zeros(svg.svg_row_similarity_workspace_bytes(s), dtype=torch.uint8, device=DEV)
    score = svg.svg_row_similarity(q.to(DEV), k.to(DEV), s, scale, workspace=ws).cpu().numpy()
    torch.cuda.synchronize()
    pats = ws[: 2 * F * Hs * N * 4].view(torch.float32).view(2, F * Hs, N).cpu().numpy()
    for h in range(2):
        qh, kh = q[0, h].float().numpy(), k[0, h].float().numpy()
        ref, eps = _pattern_bound(qh, kh, scale, Ws, range(F * Hs))
        assert (np.abs(pats[h] - ref) <= eps * ref + 1e-30).all(), f"head {h} patterns"
        want = O.row_similarity(qh, kh, scale, F, Hs, Ws)
        assert abs(score[h] - want) <= 4.1 * eps + 1e-9, (h, score[h], want, eps)


def test_row_similarity_closed_forms():
    banner("row similarity closed forms")
    F, Hs, Ws, D = 2, 4, 8, 64
    N = F * Hs * Ws
    rng = np.random.default_rng(41)
    # uniform attention: every row has the same pattern
    k = torch.from_numpy(rng.standard_normal((1, 2, N, D))).to(torch.bfloat16)
    q = torch.zeros_like(k)
    # rows attending to their own orthonormal key direction: disjoint patterns
    U_ = np.linalg.qr(rng.standard_normal((D, D)))[0][:, :F * Hs].T
    rows = np.repeat(np.arange(F * Hs), Ws)
    q[0, 1] = torch.from_numpy(U_[rows] * 60.0).to(torch.bfloat16)
    k[0, 1] = torch.from_numpy(U_[rows]).to(torch.bfloat16)
    s = svg.Shape(1, 2, N, D, F, Hs, Ws, 64)
    score = svg.svg_row_similarity(q.to(DEV), k.to(DEV), s, 1.0).cpu().numpy()
    torch.cuda.synchronize()
    assert abs(score[0] - 1.0) < 1e-6 and abs(score[1]) < 1e-6, score


def test_row_similarity_is_deterministic():
    q, k = _qk(1, 2, 700, 128, seed=43)
    s = svg.Shape(1, 2, 700, 128, 3, 5, 40, 128)
    a = svg.svg_row_similarity(q.to(DEV), k.to(DEV), s, 0.09)
    b = svg.svg_row_similarity(q.to(DEV), k.to(DEV), s, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_row_similarity_full_wan_shape_sampled(workload_inputs):
    # two heads of the Wan 720p layer: each row pattern sums to Ws (its queries'
    # weights sum to 1 each), sampled rows match the oracle, scores lie in [0, 1]
    banner("row similarity wan720p sampled")
    w, q, k, v, cls = workload_inputs("wan720p")
    heads = [int(np.nonzero(cls == 0)[0][0]), int(np.nonzero(cls == 1)[0][0])]
    qs = q[:, heads].contiguous()
    ks = k[:, heads].contiguous()
    s = svg.Shape(1, 2, w.N, w.D, w.F, w.Hs, w.Ws, w.block)
    ws = torch.empty(svg.svg_row_similarity_workspace_bytes(s), dtype=torch.uint8, device=DEV)
    score = svg.svg_row_similarity(qs.to(DEV), ks.to(DEV), s, w.scale, workspace=ws).cpu().numpy()
    rows_n = w.F * w.Hs
    pats = ws[: 2 * rows_n * w.N * 4].view(torch.float32).view(2, rows_n, w.N)
    sums = pats.double().sum(2).cpu().numpy()
    torch.cuda.synchronize()
    assert ((score >= 0) & (score <= 1 + 1e-9)).all(), score
    sample = [0, w.Hs - 1, rows_n // 2, rows_n - 1]
    for a in range(2):
        ref, eps = _pattern_bound(qs[0, a].float().numpy(), ks[0, a].float().numpy(), w.scale, w.Ws, sample)
        got = pats[a, sample].cpu().numpy()
        assert (np.abs(got - ref) <= eps * ref + 1e-30).all(), f"head {heads[a]}"
        np.testing.assert_allclose(sums[a], w.Ws, rtol=eps)
