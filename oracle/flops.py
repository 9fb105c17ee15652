"""Algorithmic work of block-masked attention.

Each kept block pair (r, c) costs one q k^T product and one p v product over
the tokens actually present: 2 * D multiply-adds per (query, key) pair, i.e.
4 * D floating-point operations.  Tokens past the sequence end do not exist
and are not counted.
"""
import numpy as np


def kept_pairs(M: np.ndarray, N: int, B: int) -> int:
    """Number of (query, key) token pairs inside the kept blocks of mask M."""
    nB = M.shape[0]
    sizes = np.array([min(N, (b + 1) * B) - b * B for b in range(nB)], dtype=np.int64)
    return int(sizes @ (M.astype(np.int64) @ sizes))


def algorithmic_flops(masks_per_head, N: int, B: int, D: int) -> int:
    """4 * D * kept pairs summed over heads (list of per-head masks)."""
    return sum(4 * D * kept_pairs(M, N, B) for M in masks_per_head)
