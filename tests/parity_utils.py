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
# profiler errors: relative deviation of each mask's error from the oracle's
PROFILE_ERR_REL = 5e-2


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
