"""Pins of the oracle's FP8 (E4M3) main-cache entries (oracle/fp8.py) against the OCP E4M3
definition and a brute-force nearest-value search: hand-worked codes, every code's round trip,
random and midpoint values against the table search, bf16 exactness and the 576-byte layout
("DeepSeek V4-Flash: The Cost of Deciding What to Read", "What the cache costs, checked
four ways": 64 bf16 RoPE dims + 448 FP8 dims = 576 bytes)."""
import numpy as np
import pytest

from oracle import fp8

FINITE = np.array([c for c in range(256) if not ((c & 0x7F) == 0x7F)], dtype=np.int64)


def brute(x: float) -> int:
    """Nearest finite E4M3 value by exhaustive search, ties to the even code; +0 for zero."""
    vals = fp8.E4M3_VALUES[FINITE]
    d = np.abs(vals - x)
    best = np.flatnonzero(d == d.min())
    cands = sorted({int(FINITE[i]) for i in best})
    if any(fp8.E4M3_VALUES[c] == 0 for c in cands):
        return 0
    if len(cands) == 1:
        return cands[0]
    # a tie between two adjacent values: the even code
    even = [c for c in cands if c % 2 == 0]
    assert len(even) == 1, (x, cands)
    return even[0]


@pytest.mark.parametrize("x,code", [
    (1.0, 0x38), (-1.0, 0xB8), (1.5, 0x3C), (448.0, 0x7E), (-448.0, 0xFE),
    (2.0 ** -6, 0x08), (2.0 ** -9, 0x01), (7 * 2.0 ** -9, 0x07), (0.0, 0x00), (-0.0, 0x00),
    (1000.0, 0x7E), (-1000.0, 0xFE), (464.0, 0x7E), (2.0 ** -11, 0x00), (2.0 ** -10, 0x00),
    (-2.0 ** -10, 0x00), (1.5 * 2.0 ** -10, 0x01), (1.0625, 0x38), (1.1875, 0x3A),
    (7.5 * 2.0 ** -9, 0x08), (240.0, 0x77), (256.0, 0x78), (3.0, 0x44),
])
def test_hand_codes(x, code):
    """Codes worked out by hand from the bit fields (bias 7: 1.0 = 0.0111.000; 448 = 0.1111.110;
    min normal 2^-6 = 0.0001.000; subnormal m * 2^-9); 1.0625 and 1.1875 are midpoints that go
    to the even mantissa; 464 is the midpoint of 448 and the missing 480 and saturates."""
    assert int(fp8.quantize(np.array([x]))[0]) == code


def test_nan_and_max_codes():
    assert np.isnan(fp8.e4m3_value(0x7F)) and np.isnan(fp8.e4m3_value(0xFF))
    assert fp8.e4m3_value(0x7E) == 448.0 and fp8.e4m3_value(0x01) == 2.0 ** -9
    assert fp8.ENTRY_BYTES == 64 * 2 + 448 == 576


def test_every_code_round_trips():
    """decode then encode gives the same code for every finite code (-0 -> +0)."""
    vals = fp8.E4M3_VALUES[FINITE]
    got = fp8.quantize(vals).astype(np.int64)
    want = np.where(FINITE == 0x80, 0, FINITE)
    assert np.array_equal(got, want)


def test_random_and_midpoints_match_table_search():
    rng = np.random.default_rng(8)
    x = np.concatenate([
        rng.choice([-1, 1], 3000) * np.exp2(rng.uniform(-13, 10, 3000)),
        rng.normal(0, 0.05, 1000),
    ])
    pos = np.sort(np.unique(np.abs(fp8.E4M3_VALUES[FINITE])))
    mids = (pos[1:] + pos[:-1]) / 2
    x = np.concatenate([x, mids, -mids, [500.0, 479.9, 480.0, 1e9, 2.0 ** -20]])
    got = fp8.quantize(x)
    for xi, gi in zip(x, got):
        assert int(gi) == brute(float(xi)), xi


def test_values_are_exact_in_bf16():
    """Every finite E4M3 value is a bf16 value: the cached entry is exact in bf16."""
    v = fp8.E4M3_VALUES[FINITE].astype(np.float32)
    b = (v.view(np.uint32) & 0xFFFF0000).view(np.float32)
    assert np.array_equal(v, b)


def test_entry_layout():
    rng = np.random.default_rng(3)
    v = np.zeros((2, 512))
    v[:, :448] = fp8.E4M3_VALUES[rng.choice(FINITE, (2, 448))]
    v[:, 448:] = rng.normal(0, 1, (2, 64)).astype(np.float32)
    v[:, 448:] = (v[:, 448:].astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
    v[0, 448] = 1.0    # bf16 0x3F80 -> bytes 0x80, 0x3F
    v[0, 0] = -1.5     # E4M3 0xBC
    e = fp8.encode_entries(v)
    assert e.shape == (2, 576) and e.dtype == np.uint8
    assert e[0, 0] == 0xBC and e[0, 448] == 0x80 and e[0, 449] == 0x3F
    assert np.array_equal(fp8.decode_entries(e), np.where(v == 0, 0.0, v))
    # the FP8 part of a cached entry is the nearest E4M3 value of the stored one
    w = rng.normal(0, 1, (3, 512))
    c = fp8.cached_entries(w)
    for i in range(3):
        for j in (0, 100, 447):
            assert c[i, j] == fp8.e4m3_value(brute(w[i, j]))
