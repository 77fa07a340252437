"""Pins of the oracle's FP4 main-cache entries (oracle/kv_fp4.py): blocks worked by hand, the
figures the page prints (largest magnitude 2,688, 4.5 bits per element, 288 bytes per entry:
"DeepSeek-V4.1-Flash's KV-Cache Compression, Checked Down to the Byte", section 4, Cell 3),
round trips of grid values, the nearest-value property against a brute force over every
representable value of the block, and the entry layout."""
import json
import pathlib

import numpy as np
import pytest

from oracle import fp8, kv_fp4, mx

GOLDEN = json.loads((pathlib.Path(__file__).parent / "golden" / "pages_printed_values.json")
                    .read_text())["fp4_main_kv"]


def block(vals):
    x = np.zeros(512)
    x[:len(vals)] = vals
    return x


def test_printed_figures():
    # largest magnitude: E2M1's 6 times E4M3's 448; 4 bits + one scale byte per 16 channels
    assert kv_fp4.E2M1_MAX * fp8.E4M3_MAX == GOLDEN["representable_max_printed"]
    assert 4 + 8 / kv_fp4.BLOCK == GOLDEN["bits_per_element_printed"]
    assert kv_fp4.ENTRY_BYTES == GOLDEN["entry_bytes_printed"]
    assert kv_fp4.CODE_BYTES == GOLDEN["code_bytes_printed"]
    assert kv_fp4.N_BLOCKS == GOLDEN["scale_bytes_printed"]
    # and the oracle reaches it: a block whose maximum is 2,688 keeps it exactly
    x = block([2688.0, -2688.0, 1000.0])
    e = kv_fp4.encode_entries(x)
    assert e[256] == 0x7E                      # scale 448
    assert kv_fp4.decode_entries(e)[:3].tolist() == [2688.0, -2688.0, 896.0]   # 1000/448 -> 2


def test_hand_worked_power_of_two_scale():
    # amax 3 -> 3 / 6 = 0.5 (E4M3 code 0x30); elements x / 0.5 = 2x:
    # 3 -> 6 (code 7); 0.2 -> 0.4 -> 0.5 (1); 0.125 -> 0.25, tie 0 / 0.5 -> 0 (even code 0);
    # 0.375 -> 0.75, tie 0.5 / 1 -> 1 (code 2); -1 -> -2 (8 | 4); 1.25 -> 2.5, tie 2 / 3 -> 2
    # (4); 1.75 -> 3.5, tie 3 / 4 -> 4 (6); 2.5 -> 5, tie 4 / 6 -> 4 (6); -0.01 -> 0 (code 0)
    x = block([3.0, 0.2, 0.125, 0.375, -1.0, 1.25, 1.75, 2.5, -0.01])
    codes, sc = kv_fp4.quantize(x)
    assert sc[0] == 0x30 and fp8.e4m3_value(0x30) == 0.5
    assert codes[:9].tolist() == [7, 1, 0, 2, 12, 4, 6, 6, 0]
    assert np.all(codes[9:] == 0) and np.all(sc[1:] == 0)
    assert kv_fp4.dequantize(codes, sc)[:9].tolist() == [3.0, 0.25, 0.0, 0.5, -1.0, 1.0, 2.0,
                                                         2.0, 0.0]


def test_hand_worked_scale_with_mantissa():
    # amax 7.5 -> 7.5 / 6 = 1.25, an E4M3 value (exponent 0, mantissa 2: code 0x3A); the power-
    # of-two MX rule would have chosen 2^(floor(log2 7.5) - 2) = 1 instead
    # 1.25 -> 1 (2); 0.9375 -> 0.75, tie 0.5 / 1 -> 1 (2); 3 -> 2.4 -> 2 (4);
    # -4.4 -> -3.52 -> -4 (8 | 6); 6.5 -> 5.2 -> 6 (7)
    x = block([7.5, 1.25, 0.9375, 3.0, -4.4, 6.5])
    codes, sc = kv_fp4.quantize(x)
    assert sc[0] == 0x3A and fp8.e4m3_value(0x3A) == 1.25
    assert codes[:6].tolist() == [7, 2, 2, 4, 14, 7]
    assert kv_fp4.dequantize(codes, sc)[:6].tolist() == [7.5, 1.25, 1.25, 2.5, -5.0, 7.5]


def test_scale_rounding_and_its_ties():
    # 6.6 / 6 = 1.1: nearest E4M3 is 1.125 (code 0x39), then 6.6 / 1.125 = 5.87 -> 6
    codes, sc = kv_fp4.quantize(block([6.6]))
    assert sc[0] == 0x39 and codes[0] == 7
    # 6.375 / 6 = 1.0625, halfway between 1 (code 0x38) and 1.125 (0x39): the even code, 1;
    # then 6.375 / 1 = 6.375 lies past 6 and saturates to 6
    codes, sc = kv_fp4.quantize(block([6.375]))
    assert sc[0] == 0x38 and codes[0] == 7
    # past E4M3's 448: the scale saturates, the elements saturate at 6 x 448
    codes, sc = kv_fp4.quantize(block([6000.0, -3000.0, 100.0]))
    assert sc[0] == 0x7E and codes[:3].tolist() == [7, 15, 0]   # 100 / 448 = 0.22 -> 0


def test_tiny_and_zero_blocks():
    # amax / 6 = 2^-10, halfway between 0 and the smallest subnormal 2^-9: the even code 0,
    # a zero scale, and every element code 0
    codes, sc = kv_fp4.quantize(block([6 * 2.0 ** -10, -2.0 ** -10]))
    assert sc[0] == 0 and not codes.any()
    # just above: scale 2^-9 (code 0x01), 6.06 x 2^-10 / 2^-9 = 3.03 -> 3 (code 5)
    codes, sc = kv_fp4.quantize(block([6.06 * 2.0 ** -10]))
    assert sc[0] == 0x01 and codes[0] == 5
    codes, sc = kv_fp4.quantize(np.zeros((2, 512)))
    assert not codes.any() and not sc.any()
    e = kv_fp4.encode_entries(np.zeros(512))
    assert not e.any() and np.array_equal(kv_fp4.decode_entries(e), np.zeros(512))


def test_layout_nibbles_and_scale_bytes():
    # channel 2i in the low nibble of byte i; block g's scale at byte 256 + g
    x = np.zeros(512)
    x[0], x[1] = 6.0, -3.0             # block 0: scale 1, codes 7 and 8 | 5
    x[16 * 5 + 3] = 0.75               # block 5: 0.75 / 6 = 0.125 = 2^-3 (code 4 << 3), element 6 -> 7
    e = kv_fp4.encode_entries(x)
    assert e.shape == (288,)
    assert e[0] == (7 | (13 << 4))
    assert e[256] == 0x38 and e[256 + 5] == 0x20 and fp8.e4m3_value(0x20) == 0.125
    assert e[(16 * 5 + 3) // 2] == 7 << 4    # odd channel: high nibble
    assert np.count_nonzero(e[256:]) == 2


def test_grid_values_round_trip_exactly():
    # values element x scale with a +-6 element in every block come back unchanged
    g = np.random.default_rng(11)
    s = g.choice(np.arange(1, 0x7F), size=(5, 32))     # finite, non-zero scale codes
    c = g.integers(0, 16, size=(5, 512)).astype(np.uint8)
    c[c == 8] = 0                                       # no negative zero
    c[:, ::16] = np.where(g.random((5, 32)) < 0.5, 7, 15)
    v = kv_fp4.dequantize(c, s.astype(np.uint8))
    codes, sc = kv_fp4.quantize(v)
    assert np.array_equal(sc, s) and np.array_equal(codes, c)
    assert np.array_equal(kv_fp4.cached_entries(v), v)


def test_nearest_value_against_brute_force():
    # every element of a random block lands on the value of the block's grid (its scale times
    # each signed E2M1 value) nearest to it, the even code on a tie; the scale is the E4M3
    # value nearest to amax / 6. Brute force over all candidates, one element at a time.
    g = np.random.default_rng(12)
    x = g.standard_normal((3, 512)) * np.exp(g.uniform(-6, 4, size=(3, 1)))
    x[0, :16] = 0.0
    x[1, 16:32] *= 1e-4
    codes, sc = kv_fp4.quantize(x)
    finite = [c for c in range(256) if not np.isnan(fp8.e4m3_value(c)) and c < 0x80]
    for r in range(3):
        for b in range(32):
            blk = x[r, 16 * b:16 * b + 16]
            amax = np.abs(blk).max()
            dist = [abs(fp8.e4m3_value(c) - amax / 6) for c in finite]
            best = [c for c, d in zip(finite, dist) if d == min(dist)]
            want_sc = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
            if amax / 6 > 448:
                want_sc = 0x7E
            assert sc[r, b] == want_sc
            s = fp8.e4m3_value(int(sc[r, b]))
            for j in range(16):
                if s == 0:
                    assert codes[r, 16 * b + j] == 0
                    continue
                xv = blk[j]
                d = [abs(mx.e2m1_value(c) * s - xv) for c in range(16)]
                cands = [c for c in range(16) if d[c] == min(d)]
                want = [c for c in cands if (c & 1) == 0 and c != 8] or cands
                got = int(codes[r, 16 * b + j])
                assert mx.e2m1_value(got) * s == mx.e2m1_value(want[0]) * s, (r, b, j, xv)
                assert got != 8                      # never a negative zero


def test_cached_values_are_bf16_values():
    # element x scale carries at most 6 significant bits: exact in bf16 (and fp32)
    g = np.random.default_rng(13)
    v = kv_fp4.cached_entries(g.standard_normal((4, 512)) * 3)
    f32 = v.astype(np.float32)
    bits = f32.view(np.uint32)
    assert np.array_equal(f32.astype(np.float64), v)
    assert not np.any(bits & 0xFFFF)


def test_error_bound():
    # |x - cached| <= half the widest E2M1 gap (2, between 4 and 6) times the scale, and the
    # scale is within half an E4M3 step of amax / 6: a relative bound over each block's amax
    g = np.random.default_rng(14)
    x = g.standard_normal((8, 512))
    c = kv_fp4.cached_entries(x)
    blk = np.abs(x).reshape(8, 32, 16).max(axis=-1)
    err = np.abs(x - c).reshape(8, 32, 16).max(axis=-1)
    assert np.all(err <= blk / 6 * (1 + 1 / 16) * 1.0 + 1e-12)
