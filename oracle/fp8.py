"""FP8 (e4m3) quantization for the FP8 attention variant, in float64 / float32.

[CalibAtt] section 3.3 puts FP8 on the critical path ("mixed precision": the
two attention products in FP8, the softmax in higher precision) without
fixing the format details; the plainest reading is the OCP 8-bit floating
point format E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
subnormals; no infinities; the all-ones exponent and mantissa is NaN, so the
largest finite value is 1.75 * 2^8 = 448), rounded to nearest, ties to even.

Scaling (reading): one factor per (tensor, head).  amax = max |x| over the
head's N x D elements (exact: the inputs are bf16); inv = 448 / amax in
float32 (1 when amax = 0); each element is taken to float32, multiplied by inv
in float32 and rounded to E4M3; its value is code / inv.  The dequantization
factor the attention uses is d = amax / 448 in float32 (1 when amax = 0).

TEST INFRASTRUCTURE (see the package header).
"""
import numpy as np

E4M3_MAX = 448.0
_SUB = 2.0 ** -9          # spacing of the subnormals (exponent field 0)


def e4m3_value(code) -> np.ndarray:
    """float64 value of E4M3 codes (uint8); NaN for the NaN codes."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * _SUB, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def _finite_table():
    codes = np.arange(128, dtype=np.int64)
    codes = codes[codes != 0x7F]             # the positive NaN code
    return codes, e4m3_value(codes)          # ascending: 0 .. 448


def e4m3_round(x) -> np.ndarray:
    """E4M3 code (uint8) of the nearest representable value, ties to the even
    code (the one whose mantissa's last bit is 0); the sign bit follows x's
    (a negative value that rounds to zero gives the negative zero code).  A
    value above 448 but below 464 (448 plus half its spacing of 32) is nearest
    to 448; |x| >= 464 would overflow and is refused (the scaling keeps every
    input below: amax * (448 / amax) exceeds 448 by an fp32 rounding at most)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) >= E4M3_MAX + 16.0) or np.any(np.isnan(x)):
        raise ValueError("e4m3_round: input outside the finite E4M3 range")
    codes, vals = _finite_table()
    a = np.abs(x)
    hi = np.searchsorted(vals, a, side="left")          # vals[hi] >= a
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi] & 1) == 0))
    c = np.where(pick_hi, codes[hi], codes[lo])
    return (c | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def head_scale(x):
    """(inv, d) of one head's tensor x (any float dtype): inv = 448 / amax and
    d = amax / 448 in float32, both 1 when amax = 0."""
    amax = np.float32(np.max(np.abs(np.asarray(x, dtype=np.float32))))
    if amax == 0:
        return np.float32(1.0), np.float32(1.0)
    return np.float32(E4M3_MAX) / amax, amax / np.float32(E4M3_MAX)


def quantize_head(x):
    """E4M3 codes of one head's [N, D] tensor, with its (inv, d) factors, and
    the float64 values the codes stand for (code / inv)."""
    inv, d = head_scale(x)
    y = np.asarray(x, dtype=np.float32) * inv             # float32 product, nearest even
    codes = e4m3_round(y.astype(np.float64))
    return codes, inv, d, e4m3_value(codes) / np.float64(inv)


def vt8_key_order(block: int = 128) -> np.ndarray:
    """Position of each key of a block in an FP8 V^T row: within every group
    of 64 keys the keys 8a + 4h + i (a < 8, h < 2, i < 4) go to position
    32h + 4a + i, so that each half of the group is one contiguous run of 32
    bytes (the operand layout of the 64-deep FP8 matrix product)."""
    k = np.arange(block)
    g, kk = np.divmod(k, 64)
    a, r = np.divmod(kk, 8)
    h, i = np.divmod(r, 4)
    return 64 * g + 32 * h + 4 * a + i


def vt8_blocks(codes_kv: np.ndarray, block: int = 128) -> np.ndarray:
    """uint8 [nB, D, block]: the V codes of one head (rows in the head's layout)
    transposed per key block, keys placed by vt8_key_order, keys past N zero."""
    N, D = codes_kv.shape
    nB = -(-N // block)
    pad = np.zeros((nB * block, D), np.uint8)
    pad[:N] = codes_kv
    t = pad.reshape(nB, block, D).transpose(0, 2, 1)      # [nB, D, key]
    out = np.empty_like(t)
    out[:, :, vt8_key_order(block)] = t
    return out
