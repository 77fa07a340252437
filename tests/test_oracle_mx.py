"""Pins of the MXFP4 oracle (oracle/mx.py) against the format's definition, worked by hand."""
import numpy as np
import pytest

from oracle import mx


def test_e2m1_values_from_bit_fields():
    # sign | 2 exponent bits (bias 1) | 1 mantissa bit; exponent 0 is subnormal (0.m x 2^0)
    assert list(mx.E2M1_MAGNITUDES) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert [mx.e2m1_value(c) for c in range(8, 16)] == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0,
                                                        -4.0, -6.0]


def test_hand_worked_block():
    # max |x| = 0.75 -> floor(log2 0.75) = -1 -> s = -3, scale byte 124, x / 2^s = 8 x
    x = np.zeros(32)
    x[:10] = [0.75, 0.1, 0.2, 0.03125, 0.09375, -0.3, 0.15625, 0.3125, 0.4375, -0.75]
    codes, scales = mx.quantize(x[None])
    assert scales.tolist() == [[124]]
    # 8x: 6 -> code 7; 0.8 -> 1.0 (code 2); 1.6 -> 1.5 (code 3); 0.25 tie 0 / 0.5 -> 0;
    # 0.75 tie 0.5 / 1.0 -> 1.0 (even code 2); -2.4 -> -2 (code 8 | 4); 1.25 tie 1.0 / 1.5 ->
    # 1.0; 2.5 tie 2 / 3 -> 2 (code 4); 3.5 tie 3 / 4 -> 4 (code 6); -6 -> code 15
    assert codes[0, :10].tolist() == [7, 2, 3, 0, 2, 12, 2, 4, 6, 15]
    assert np.all(codes[0, 10:] == 0)
    deq = mx.dequantize(codes, scales)[0]
    assert deq[:10].tolist() == [0.75, 0.125, 0.1875, 0.0, 0.125, -0.25, 0.125, 0.25, 0.5, -0.75]


def test_saturation_and_tie_at_five():
    # max |x| = 7.5 -> s = 0: 7.5 saturates to 6, 5 ties 4 / 6 -> 4 (even), 5.5 -> 6
    x = np.zeros(32)
    x[:3] = [7.5, 5.0, 5.5]
    codes, scales = mx.quantize(x[None])
    assert scales.tolist() == [[127]]
    assert codes[0, :3].tolist() == [7, 6, 7]


def test_zero_block_and_negative_zero():
    codes, scales = mx.quantize(np.zeros((1, 64)))
    assert scales.tolist() == [[0, 0]] and not codes.any()
    x = np.zeros(32)
    x[0], x[1] = 1.0, -0.01          # -0.01 * 4 rounds to magnitude 0: code 0, not -0
    codes, _ = mx.quantize(x[None])
    assert codes[0, 1] == 0


def test_grid_values_round_trip_exactly():
    g = np.random.default_rng(5)
    s = g.integers(-20, 20, size=(6, 4))
    c = g.integers(0, 16, size=(6, 128)).astype(np.uint8)
    c[:, ::32] = 7                    # each block holds its largest magnitude
    x = mx.dequantize(c, s + 127)
    codes, scales = mx.quantize(x)
    assert np.array_equal(scales, s + 127)
    assert np.array_equal(mx.dequantize(codes, scales), x)


def test_error_bound_and_scale_range():
    g = np.random.default_rng(6)
    x = g.standard_normal((50, 128)) * np.exp(g.standard_normal((50, 1)))
    codes, scales = mx.quantize(x)
    deq = mx.dequantize(codes, scales)
    s = np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=-1)
    v = np.abs(x) / s
    # half the gap of the E2M1 grid around v, the saturating top interval [6, 8) excepted
    half_gap = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    bound = np.where(v <= 6, half_gap, v - 6)
    assert np.all(np.abs(x - deq) <= bound * s + 1e-300)
    amax = np.abs(x).reshape(50, 4, 32).max(-1)
    ratio = amax / 2.0 ** (scales.astype(np.float64) - 127)
    assert np.all((ratio >= 4) & (ratio < 8))


def test_monotone_within_a_block():
    x = np.linspace(-1.0, 1.0, 32)
    codes, scales = mx.quantize(x[None])
    d = mx.dequantize(codes, scales)[0]
    assert np.all(np.diff(d) >= 0)


def test_pack_nibble_order():
    c = np.arange(16, dtype=np.uint8)[None]
    p = mx.pack(c)
    assert p.tolist() == [[0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]]
    assert np.array_equal(mx.unpack(p), c)


def test_quantize_matches_the_scalar_rounding():
    # every element through round_e2m1 one by one: random values and every tie of the grid
    g = np.random.default_rng(7)
    x = g.standard_normal((4, 128)) * np.exp(2 * g.standard_normal((4, 1)))
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    x[:, 1:17] = np.concatenate([ties, -ties]) * 2.0 ** (mx.shared_exponent(x[0, :32]))
    x[:, 0] = 7.0 * 2.0 ** mx.shared_exponent(x[0, :32])      # the first block's maximum
    codes, scales = mx.quantize(x)
    for i in range(x.shape[0]):
        for b in range(4):
            blk = x[i, 32 * b:32 * b + 32]
            s = mx.shared_exponent(blk)
            assert scales[i, b] == s + 127
            assert [int(c) for c in codes[i, 32 * b:32 * b + 32]] == \
                [mx.round_e2m1(v * 2.0 ** -s) for v in blk]
