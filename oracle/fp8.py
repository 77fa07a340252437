"""FP8 (E4M3) storage of the main KV entries, float64 oracle -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this module; the product path never does.

"DeepSeek V4-Flash: The Cost of Deciding What to Read", section "What the cache costs, checked four
ways": the rotary part of a head is exactly its last 64 dimensions, those are kept in bf16
and the rest in FP8, so one shared key/value entry of head dimension 512 takes 64 * 2 + 448 =
576 bytes; section "The indexer is O(n), and that is the ceiling": the main attention runs
in FP8.

Readings taken (the pages fix the byte count, not the element format):
  * FP8 is the OCP E4M3 format ("fn": 1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
    infinities; S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448;
    exponent field 0 holds the subnormals m * 2^-9).
  * No scale: 576 bytes leave no room for one, and the entries the cache holds are RMS-
    normalised per head, well inside E4M3's range.
  * A value is rounded to the nearest E4M3 value, ties to the even code (mantissa bit 0);
    magnitudes past 448 go to 448 (saturation; there is no infinity to go to); a zero
    magnitude is always code 0x00 (never -0).
  * Entry layout: bytes 0 .. 447 are the E4M3 codes of channels 0 .. 447; bytes 448 .. 575
    are channels 448 .. 511 as bf16 (little-endian, nearest-even from the stored value).
  * Which value is quantised: the entry as the path stores it in its dtype (bf16), as for the
    MXFP4 indexer keys.
Every E4M3 value is exactly representable in bf16 (3 mantissa bits, exponents -9 .. 8), so an
entry's cached value is exact in bf16 as well.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_BIAS = 7
ENTRY_DIM = 512
ROPE_DIM = 64
NOPE_DIM = ENTRY_DIM - ROPE_DIM          # 448 channels in FP8
ENTRY_BYTES = NOPE_DIM + 2 * ROPE_DIM    # 576


def e4m3_value(code: int) -> float:
    """Value of an 8-bit E4M3 code from its bit fields (NaN for S.1111.111)."""
    s, e, m = (code >> 7) & 1, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = (m / 8.0) * 2.0 ** (1 - E4M3_BIAS) if e == 0 else 2.0 ** (e - E4M3_BIAS) * (1 + m / 8.0)
    return -mag if s else mag


E4M3_VALUES = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def quantize(x) -> np.ndarray:
    """E4M3 codes (uint8) of x, element by element, by the rules in the module docstring.

    The grid spacing at |x| is 2^(e - 3) with e = floor(log2 |x|) in the normal range and
    e = -6 below it (subnormal spacing 2^-9); |x| / spacing is rounded half-to-even."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, ex = np.frexp(np.maximum(a, 2.0 ** -6))     # a = f * 2^ex, f in [0.5, 1)
    ulp = np.ldexp(1.0, (ex - 1) - 3)
    q = np.minimum(np.rint(a / ulp) * ulp, E4M3_MAX)
    # code of the magnitude q (q is on the grid)
    _, eq = np.frexp(np.maximum(q, 2.0 ** -6))
    e = eq - 1                                       # binade of q (>= -6)
    normal = q >= 2.0 ** -6
    m_norm = np.rint(np.ldexp(q, -(e - 3))) - 8      # 0 .. 7
    code_norm = ((e + E4M3_BIAS) << 3) + m_norm
    code_sub = np.rint(np.ldexp(q, 9))               # 0 .. 7
    code = np.where(normal, code_norm, code_sub).astype(np.int64)
    neg = (x < 0) & (q > 0)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def dequantize(codes) -> np.ndarray:
    """Values (float64) of E4M3 codes."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def _bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of v (rounded to fp32, then to bf16 nearest-even)."""
    u = np.asarray(v, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def encode_entries(v) -> np.ndarray:
    """Entries [..., 512] -> bytes [..., 576]: E4M3 codes of channels 0..447, then channels
    448..511 as little-endian bf16."""
    v = np.asarray(v, dtype=np.float64)
    assert v.shape[-1] == ENTRY_DIM
    out = np.empty(v.shape[:-1] + (ENTRY_BYTES,), dtype=np.uint8)
    out[..., :NOPE_DIM] = quantize(v[..., :NOPE_DIM])
    b = _bf16_bits(v[..., NOPE_DIM:])
    out[..., NOPE_DIM::2] = (b & 0xFF).astype(np.uint8)
    out[..., NOPE_DIM + 1::2] = (b >> 8).astype(np.uint8)
    return out


def decode_entries(e) -> np.ndarray:
    """Bytes [..., 576] -> the entries' values [..., 512] (float64)."""
    e = np.asarray(e, dtype=np.uint8)
    assert e.shape[-1] == ENTRY_BYTES
    out = np.empty(e.shape[:-1] + (ENTRY_DIM,), dtype=np.float64)
    out[..., :NOPE_DIM] = dequantize(e[..., :NOPE_DIM])
    bits = e[..., NOPE_DIM::2].astype(np.uint32) | (e[..., NOPE_DIM + 1::2].astype(np.uint32) << 8)
    out[..., NOPE_DIM:] = (bits << 16).view(np.float32).astype(np.float64)
    return out


def cached_entries(v) -> np.ndarray:
    """The value an FP8 cache holds for entries v (already in the path's dtype)."""
    return decode_entries(encode_entries(v))
