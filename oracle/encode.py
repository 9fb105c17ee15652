"""Bitmap and skip-list encoding of block masks ([CalibAtt] section 3.3).

The article stores each mask as a bitmap (one bit per block instead of a
32-bit entry, hence 32x smaller) and precomputes, per query-block row, a skip
list of contiguous kept-block intervals so the kernel visits kept blocks only.

Readings (the pages give no format):
* bitmap: uint32 words, row-major [mask][query block][word]; key block c is
  bit c % 32 of word c // 32 (least significant bit first); padding bits are 0.
* skip list: CSR.  row_ptr[m*nQB + r] .. row_ptr[m*nQB + r + 1] index the
  intervals of row r of mask m; each interval is an int32 pair [start, end)
  of key blocks.  Intervals of a row are ascending, disjoint and maximal (a
  kept block never touches the next interval).  Empty rows have no interval.
"""
import numpy as np


def iv_capacity(n_masks: int, n_qb: int, n_kb: int) -> int:
    """Worst-case interval count: every row alternates kept / skipped blocks."""
    return n_masks * n_qb * ((n_kb + 1) // 2)


def _row_runs(row: np.ndarray):
    """Maximal runs of nonzero entries of a 1-D row as (starts, ends)."""
    edge = np.diff(np.concatenate(([0], (row != 0).astype(np.int8), [0])))
    return np.nonzero(edge == 1)[0], np.nonzero(edge == -1)[0]


def encode_masks(M: np.ndarray):
    """M uint8 [n_masks, nQB, nKB] -> (bitmap uint32 [n_masks, nQB, W], row_ptr int32
    [n_masks*nQB + 1], iv int32 [n_iv, 2]) with W = ceil(nKB / 32)."""
    M = np.asarray(M)
    n_masks, nQB, nKB = M.shape
    W = -(-nKB // 32)
    bitmap = np.zeros((n_masks, nQB, W), dtype=np.uint32)
    row_ptr = np.zeros(n_masks * nQB + 1, dtype=np.int32)
    ivs = []
    for m in range(n_masks):
        for r in range(nQB):
            row = M[m, r]
            bits = np.zeros(W * 32, dtype=np.uint8)
            bits[:nKB] = row != 0
            # packbits(little) puts element 8b+t in bit t of byte b; four bytes
            # read little-endian form word w with element 32w+t in bit t.
            bitmap[m, r] = np.packbits(bits, bitorder="little").view("<u4")
            starts, ends = _row_runs(row)
            ivs.extend(zip(starts.tolist(), ends.tolist()))
            row_ptr[m * nQB + r + 1] = row_ptr[m * nQB + r] + len(starts)
    iv = np.array(ivs, dtype=np.int32).reshape(-1, 2)
    return bitmap, row_ptr, iv


def decode_masks(bitmap: np.ndarray, row_ptr: np.ndarray, iv: np.ndarray, nKB: int):
    """Rebuild the dense masks twice, from the bitmap and from the skip list."""
    n_masks, nQB, W = bitmap.shape
    c = np.arange(nKB)
    from_bits = ((bitmap[:, :, c // 32] >> (c % 32).astype(np.uint32)) & 1).astype(np.uint8)
    from_iv = np.zeros((n_masks, nQB, nKB), dtype=np.uint8)
    for m in range(n_masks):
        for r in range(nQB):
            for j in range(row_ptr[m * nQB + r], row_ptr[m * nQB + r + 1]):
                from_iv[m, r, iv[j, 0]:iv[j, 1]] = 1
    return from_bits, from_iv
