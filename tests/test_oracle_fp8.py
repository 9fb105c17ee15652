"""Pins of the oracle's E4M3 quantizer and FP8 layouts (CPU only).

The format facts checked here are those of the OCP 8-bit floating point
specification's E4M3: bias 7, 3 mantissa bits, subnormals of spacing 2^-9,
largest finite value 448, one NaN mantissa pattern per sign, no infinities."""
import numpy as np
import pytest

import oracle.fp8 as F8
import oracle as O


def test_code_table_closed_forms():
    v = F8.e4m3_value(np.arange(256))
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0 ** -9                       # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9                   # largest subnormal
    assert v[0x08] == 2.0 ** -6                       # smallest normal
    assert v[0x38] == 1.0 and v[0x40] == 2.0 and v[0x3C] == 1.5
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0     # largest finite
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    finite = v[:127]
    assert np.all(np.diff(finite) > 0)                # codes 0..126 ascend
    assert np.array_equal(v[128:255], -v[:127])


def test_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], np.uint8)
    assert np.array_equal(F8.e4m3_round(F8.e4m3_value(codes)), codes)


def test_ties_go_to_even_codes():
    # halfway between 1.0 (0x38) and 1.125 (0x39): even code 0x38
    assert F8.e4m3_round(1.0625) == 0x38
    # halfway between 1.125 (0x39) and 1.25 (0x3A): 0x3A
    assert F8.e4m3_round(1.1875) == 0x3A
    # subnormals: 0.5 * 2^-9 -> 0 (even), 1.5 * 2^-9 -> 2 * 2^-9, 2.5 * 2^-9 -> 2 * 2^-9
    assert F8.e4m3_round(0.5 * 2.0 ** -9) == 0x00
    assert F8.e4m3_round(1.5 * 2.0 ** -9) == 0x02
    assert F8.e4m3_round(2.5 * 2.0 ** -9) == 0x02
    # between the largest subnormal and the smallest normal: 7.5 * 2^-9 -> 2^-6 (code 8, even)
    assert F8.e4m3_round(7.5 * 2.0 ** -9) == 0x08
    # 440 is halfway between 416 (0x7D) and 448 (0x7E): even code 0x7E
    assert F8.e4m3_round(440.0) == 0x7E
    assert F8.e4m3_round(-1.0625) == 0xB8
    assert F8.e4m3_round(-1e-6) == 0x80


def test_rounding_is_nearest_against_brute_force():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-448, 448, 2000), rng.uniform(-0.05, 0.05, 2000),
                        rng.normal(0, 3, 2000)])
    x = np.clip(x, -448, 448)
    c = F8.e4m3_round(x)
    table = F8.e4m3_value(np.array([k for k in range(256) if k not in (0x7F, 0xFF)]))
    best = np.min(np.abs(x[:, None] - table[None, :]), axis=1)
    assert np.all(np.abs(F8.e4m3_value(c) - x) == best)
    # above the largest finite value but nearer to it than to the overflow point
    assert F8.e4m3_round(448.0 * (1 + 2.0 ** -23)) == 0x7E and F8.e4m3_round(463.9) == 0x7E
    assert F8.e4m3_round(-449.0) == 0xFE
    with pytest.raises(ValueError):
        F8.e4m3_round(464.0)


def test_head_scale_maps_amax_to_448():
    rng = np.random.default_rng(4)
    x = rng.normal(0, 2, (300, 64)).astype(np.float32)
    codes, inv, d, val = F8.quantize_head(x)
    assert np.max(np.abs(F8.e4m3_value(codes))) == 448.0
    assert inv == np.float32(448.0) / np.float32(np.max(np.abs(x)))
    assert d == np.float32(np.max(np.abs(x))) / np.float32(448.0)
    # relative error of every normal-range value is at most 2^-4
    big = np.abs(val) >= 2.0 ** -6 / inv
    assert np.all(np.abs(val - x)[big] <= 2.0 ** -4 * np.abs(x)[big] * (1 + 1e-6))
    z = F8.quantize_head(np.zeros((4, 8), np.float32))
    assert z[1] == 1.0 and z[2] == 1.0 and not z[0].any()


def test_quantize_head_amax_product_rounding():
    """amax * inv can exceed 448 by one fp32 rounding; it still maps to 448."""
    for amax in (3.0, 5.1, 93.21290588, 119.2258072, 0.37):
        x = np.array([[amax, -amax / 3, 0.0]], np.float32)
        codes = F8.quantize_head(x)[0]
        assert codes[0, 0] == 0x7E


def test_vt8_layout_halves_are_contiguous_runs():
    pos = F8.vt8_key_order(128)
    assert sorted(pos.tolist()) == list(range(128))
    # keys 8a + 4h + i of a 64-key group sit at 32h + 4a + i
    for key in (0, 3, 4, 7, 8, 12, 60, 63, 64, 68, 127):
        g, kk = divmod(key, 64)
        a, r = divmod(kk, 8)
        h, i = divmod(r, 4)
        assert pos[key] == 64 * g + 32 * h + 4 * a + i
    N, D = 200, 4
    codes = (np.arange(N * D) % 251).astype(np.uint8).reshape(N, D)
    vt = F8.vt8_blocks(codes)
    assert vt.shape == (2, D, 128)
    for key in (0, 5, 77, 127, 128, 199):
        b, j = divmod(key, 128)
        assert np.array_equal(vt[b, :, pos[j]], codes[key])
    assert not vt[1, :, pos[np.arange(72, 128)]].any()      # keys past N are zero
