"""FP4 storage of the main KV entries (V4.1's 288-byte entry), float64 oracle -- TEST
INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this module; the product path never does.

"DeepSeek-V4.1-Flash's KV-Cache Compression, Checked Down to the Byte", section 4 ("FP4: the norm
argument, and hunting the 890-byte ledger", Cell 3 "FP4 range analysis"): the main KV cache holds
E2M1 elements with one E4M3 scale per 16 channels and no second-level global scale; a 512-channel
entry takes 512 x 0.5 + 512 / 16 = 288 bytes. The "DeepSeek-V4.1-Flash" interactive study,
"FP4 main KV" and "Reconstruct the 890-byte global cache": the whole 512-channel latent is
quantised after RoPE (256 packed bytes + 32 E4M3 scales), and attention dequantises the cached
values before it uses them (FP4 is a storage format here, not a compute format).

Readings taken (the pages fix the element and scale formats and the byte count, not the
rounding or the layout):
  * E2M1 as in the MXFP4 indexer keys (oracle/mx.py): sign, 2 exponent bits (bias 1), 1
    mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. E4M3 as in the FP8 entries
    (oracle/fp8.py): OCP "fn", largest finite 448, subnormals m * 2^-9.
  * Block scale: the E4M3 value nearest to amax / 6 (amax = the block's largest magnitude, 6 =
    E2M1's largest magnitude: the block maximum lands on the top of the element grid, the
    convention of the NVFP4 scheme the page says the format follows), ties to the even code,
    past 448 to 448. A block whose scale rounds to 0 (amax / 6 at most 2^-10, half the smallest
    subnormal) stores the scale code 0 and all element codes 0.
  * Elements: x / scale rounded to the nearest E2M1 magnitude, ties to the even code,
    magnitudes past 6 to 6 (the scale may round below amax / 6, or saturate); the sign is x's,
    except that a zero magnitude is always code 0.
  * Entry layout: bytes 0 .. 255 hold the element codes, channel 2i in the low nibble of byte i
    (as the MXFP4 indexer keys); bytes 256 .. 287 the scale codes, byte 256 + g for channels
    16 g .. 16 g + 15.
  * Which value is quantised: the entry as the path stores it in its dtype (bf16), after the
    per-head RMSNorm and RoPE the path applies to it, as for the FP8 entries.
A cached value, element x scale, is exact in bf16: E2M1 magnitudes carry 2 significant bits and
E4M3 values 4, so a product carries at most 6, with magnitudes between 2^-10 and 6 x 448 = 2,688.
"""
from __future__ import annotations

import numpy as np

from . import fp8, mx

ENTRY_DIM = 512
BLOCK = 16
N_BLOCKS = ENTRY_DIM // BLOCK            # 32 scales
CODE_BYTES = ENTRY_DIM // 2              # 256
ENTRY_BYTES = CODE_BYTES + N_BLOCKS      # 288
E2M1_MAX = 6.0

E2M1_VALUES = np.array([mx.e2m1_value(c) for c in range(16)], dtype=np.float64)


def block_scale_codes(amax) -> np.ndarray:
    """E4M3 codes of the block scales: amax / 6 rounded to the nearest E4M3 value (ties to the
    even code, saturating at 448; a zero magnitude is code 0). amax >= 0."""
    return fp8.quantize(np.asarray(amax, dtype=np.float64) / E2M1_MAX)


MIDPOINTS = (mx.E2M1_MAGNITUDES[:-1] + mx.E2M1_MAGNITUDES[1:]) / 2   # 0.25, 0.75, ..., 5


def nearest_e2m1(y) -> np.ndarray:
    """E2M1 codes of y, element by element: the nearest magnitude, ties to the even code,
    past 6 to 6, the sign of y (a zero magnitude is code 0). Between two adjacent magnitudes
    the nearer one is decided by their midpoint, so the code of |y| is the number of midpoints
    it has reached; on a midpoint (a tie) the count must stop at the even code of the two, so
    the midpoints whose upper neighbour has an even code (0.75, 1.75, 3.5) count once reached
    and the others (0.25, 1.25, 2.5, 5) only once passed."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    c = np.zeros(a.shape, dtype=np.uint8)
    for k, mid in enumerate(MIDPOINTS):
        upper_even = (k + 1) % 2 == 0
        c += ((a >= mid) if upper_even else (a > mid)).view(np.uint8)
    return np.where((c != 0) & (y < 0), c | 8, c).astype(np.uint8)


def quantize(x) -> tuple[np.ndarray, np.ndarray]:
    """Element codes (one uint8 per channel, 0..15) and scale codes (uint8 [..., 32]) of
    entries x [..., 512], by the rules in the module docstring."""
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] == ENTRY_DIM
    rows = x.reshape(-1, N_BLOCKS, BLOCK)
    codes = np.empty(rows.shape, dtype=np.uint8)
    scodes = np.empty(rows.shape[:2], dtype=np.uint8)
    for i0 in range(0, rows.shape[0], 1 << 13):              # bounded temporaries
        blk = rows[i0:i0 + (1 << 13)]
        sc = block_scale_codes(np.abs(blk).max(axis=-1))
        s = fp8.dequantize(sc)[..., None]
        y = np.divide(blk, s, out=np.zeros_like(blk), where=s > 0)   # scale 0: every code 0
        codes[i0:i0 + blk.shape[0]] = nearest_e2m1(y)
        scodes[i0:i0 + blk.shape[0]] = sc
    return codes.reshape(x.shape), scodes.reshape(x.shape[:-1] + (N_BLOCKS,))


def dequantize(codes, scodes) -> np.ndarray:
    """Values (float64) of element codes [..., 512] under scale codes [..., 32]."""
    codes = np.asarray(codes, dtype=np.uint8)
    v = np.take(E2M1_VALUES, codes).reshape(codes.shape[:-1] + (N_BLOCKS, BLOCK))
    return (v * fp8.dequantize(scodes)[..., None]).reshape(codes.shape)


def encode_entries(v) -> np.ndarray:
    """Entries [..., 512] -> bytes [..., 288]: packed element codes, then the 32 scale codes."""
    codes, scodes = quantize(v)
    out = np.empty(codes.shape[:-1] + (ENTRY_BYTES,), dtype=np.uint8)
    out[..., :CODE_BYTES] = mx.pack(codes)
    out[..., CODE_BYTES:] = scodes
    return out


def decode_entries(e) -> np.ndarray:
    """Bytes [..., 288] -> the entries' values [..., 512] (float64)."""
    e = np.asarray(e, dtype=np.uint8)
    assert e.shape[-1] == ENTRY_BYTES
    return dequantize(mx.unpack(e[..., :CODE_BYTES]), e[..., CODE_BYTES:])


def cached_entries(v) -> np.ndarray:
    """The value an FP4 cache holds for entries v (already in the path's dtype)."""
    return decode_entries(encode_entries(v))
