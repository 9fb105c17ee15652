"""Helpers shared by the GPU parity tests (comparison metrics, case banners)."""
import sys

import numpy as np
import torch

# attention outputs: bf16 inputs, fp32 accumulation, bf16 output
ATTN_MAX_ABS = 2e-2
ATTN_REL_L2 = 5e-3
# log-sum-exp: the kernels sum the fp32 weights (only the PV product uses them
# rounded to bf16), so the error is fp32 arithmetic on the oracle's own bf16
# inputs.  Scores: the bf16 products are exact and the matrix core sums D of
# them in fp32, an error of at most about D * 2^-24 * sum_d |q_d k_d|; with
# |q|, |k| <= 2 sqrt(2 D) for the generated heads (2 u_s of norm 2 sqrt(D)
# plus noise) that is <= 128 * 6e-8 * 512 * (1/sqrt(128)) = 3.5e-4 in
# natural-log units at D = 128.  Denominator: plain fp32 sums of at most 64
# terms per lane and block, then one term per block, relative error about
# (64 + 2 n_blocks) 2^-24 <= 1e-4 for n_blocks <= 931.  exp2, the scale FMA
# and the final log2 add a few ulp.  1e-3 bounds the sum with room.  (A
# denominator of bf16-rounded weights could be off by ln(1 + 2^-8) = 3.9e-3
# on a row dominated by one weight.)
LSE_ABS = 1e-3
# profiler errors: relative deviation of each mask's error from the oracle's.
# The kernel rounds the weights of its V products to bf16 (relative 2^-9 each)
# and sums in fp32; a mask's error is a difference of two weighted means of V,
# so its relative deviation is about 2^-9 times the spread of V over that
# difference: measured at most 1.9e-3 over every head of the Wan and Hunyuan
# workloads and the constructed near-tie heads.  With every error within r of
# the oracle's, the choice agrees whenever the oracle's two errors differ by a
# factor above (1 + r) / (1 - r): 1.02 at r = 1e-2, 1.0038 at the measured
# 1.9e-3 (the near-tie test checks 1.005 and 1.01).
PROFILE_ERR_REL = 1e-2


def banner(*parts):
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def attn_errors(gpu: np.ndarray, ref: np.ndarray):
    """(max-abs, rel-L2) of a GPU output against the float64 oracle."""
    gpu = np.asarray(gpu, dtype=np.float64)
    d = gpu - ref
    return float(np.max(np.abs(d))), float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30))


def assert_attn_close(gpu, ref, what=""):
    mx, rl = attn_errors(gpu, ref)
    assert mx <= ATTN_MAX_ABS and rl <= ATTN_REL_L2, f"{what}: max-abs {mx:.3e}, rel-L2 {rl:.3e}"
    return mx, rl


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def sample_qblocks(n_blocks: int, seed: int, n: int = 32, must=()):
    """n distinct seeded query blocks (fewer if the mask has fewer), always
    with block 0, the last (ragged) block, the one before it and `must`."""
    fixed = sorted(set([0, n_blocks - 2, n_blocks - 1] + [b for b in must if 0 <= b < n_blocks]))
    fixed = [b for b in fixed if b >= 0]
    rest = np.setdiff1d(np.arange(n_blocks), fixed)
    k = max(0, min(len(rest), n - len(fixed)))
    pick = np.random.default_rng(seed).choice(rest, size=k, replace=False) if k else []
    return sorted(set(fixed) | set(int(b) for b in pick))


# FP8 variant.  The oracle takes the E4M3-rounded q, k, v (oracle.fp8); what
# remains on the GPU side is (i) the FP8 product's internal accumulation,
# measured on v_mfma_f32_32x32x64_f8f6f4 at 1.5e-4 of sum |a_i b_i| and
# bounded here by 2^-11, which moves every score by at most
# E = 2^-11 * scale * d_q d_k * sum_d |q8_d k8_d|, (ii) the weights rounded to
# E4M3 for the PV product (|dw| <= 2^-4 w in the normal range, <= min(w, 2^-10)
# below it, w relative to the row's max, whatever power of two the kernel's
# running max puts on them), (iii) bf16 rounding of the output and fp32 sums.
FP8_MMA_REL = 2.0 ** -11


def fp8_bound(qd, kd, vd, M, B, scale, qblocks, self_norm=False):
    """Per-element bound on |o_fp8 - o| and per-row bound on |lse_fp8 - lse| of
    one head (float64 [N, D] and [N]; NaN outside qblocks), o and lse being
    the oracle's attention on the dequantized q, k, v in the mask's layout.

    self_norm: the output's denominator is the matrix core's sum of the E4M3
    weights themselves (the call without LSE) instead of the fp32
    weights: o' = sum q_j v_j / sum q_j with q_j = w_j + d_j, so
    o' - o_w = sum d_j (v_j - o_w) / sum q_j, at most
    (sum |d_j| |v_j| + |o_w| sum |d_j|) / (z - sum |d_j|) (every |d_j| <= w_j
    and the row's largest weight is >= 1, so the denominator stays positive),
    each weight first moved by the score error (|d_j| <= 2^-4 w_j e^E), plus
    the matrix core's accumulation of the sum and of the product (2^-11 of
    sum q_j and of sum q_j |v_j| each, taken as 2^-10 of both terms)."""
    N, D = qd.shape
    bnd = np.full((N, D), np.nan)
    e_lse = np.full(N, np.nan)
    q_abs, k_abs = np.abs(qd), np.abs(kd)
    for r in qblocks:
        rows = slice(r * B, min(N, (r + 1) * B))
        kept = np.nonzero(M[r])[0]
        if kept.size == 0:
            bnd[rows] = 1e-6
            e_lse[rows] = 0.0
            continue
        keys = np.concatenate([np.arange(c * B, min(N, (c + 1) * B)) for c in kept])
        s = (qd[rows] @ kd[keys].T) * scale
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        z = w.sum(axis=1, keepdims=True)
        v = vd[keys]
        oo = (w @ v) / z
        # score error: the FP8 product's accumulation plus the fp32 scale factors
        E = (FP8_MMA_REL * scale * (q_abs[rows] @ k_abs[keys].T).max(axis=1, keepdims=True)
             + 2.0 ** -20 * np.abs(s).max(axis=1, keepdims=True))
        dw = np.where(w >= 2.0 ** -6, 2.0 ** -4 * w, np.maximum(2.0 ** -4 * w, np.minimum(w, 2.0 ** -10)))
        if self_norm:
            dw = dw * np.exp(E)
            zq = z - dw.sum(axis=1, keepdims=True)
            oo_w = (w @ np.abs(v)) / z
            t_p = (dw @ np.abs(v) + np.abs(oo) * dw.sum(axis=1, keepdims=True)) / zq \
                + 2.0 ** -10 * (oo_w + np.abs(oo))
        else:
            t_p = (dw @ np.abs(v)) / z
        # sum_j w_j |v_jd - o_d| / z <= sum_j w_j |v_jd| / z + |o_d|
        spread = (w @ np.abs(v)) / z + np.abs(oo)
        t_s = (np.exp(E) - 1.0) * np.exp(E) * spread
        bnd[rows] = t_p + t_s + 2.0 ** -8 * np.abs(oo) + 1e-3
        e_lse[rows] = E[:, 0] + 1e-3
    return bnd, e_lse
