"""Helpers shared by the GPU parity tests (comparison metrics, case banners)."""
import sys

import numpy as np
import torch

# attention outputs: bf16 inputs, fp32 accumulation, bf16 output
ATTN_MAX_ABS = 2e-2
ATTN_REL_L2 = 5e-3
# log-sum-exp: the kernels sum the fp32 weights (only the PV product uses them
# rounded to bf16), so the error is fp32 arithmetic on the oracle's own bf16
# inputs: the scores (D products summed in fp32 by the matrix core, relative
# error about D * 2^-24 of sum |q_i k_i|, under 1e-3 in log units at these
# sizes) and the denominator (sums of at most 64 terms per lane and block,
# then one term per block: relative error about (64 + 2 n_blocks) 2^-24 <=
# 1e-4).  2.5e-3 covers both.  (A denominator of bf16-rounded weights could
# be off by ln(1 + 2^-8) = 3.9e-3 on a row dominated by one weight.)
LSE_ABS = 2.5e-3


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
