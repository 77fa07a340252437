"""MXFP4 storage of indexer keys, float64 oracle -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this module; the product path never does.

"DeepSeek V4-Flash: The Cost of Deciding What to Read", section "What the cache costs, checked
four ways" (the indexer cache is FP4: a 128-channel indexer key takes 64 bytes) and section
"FP4, down to the index scores" (the indexer's query-key path is cached and loaded in FP4; the
MXFP4 sub-blocks are 1 x 32). Reading taken for the element and scale formats (the pages name
MXFP4 but do not spell it out; another page gives a per-16 E4M3 scale for a different cache):
the OCP microscaling definition -- E2M1 elements (1 sign, 2 exponent, 1 mantissa bit, exponent
bias 1; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) sharing one E8M0 scale 2^(s - 127) per block of
32 consecutive channels. A 128-channel key: 64 bytes of elements + 4 scale bytes.

Quantisation of one block x (the stored bf16 values, exact in float64):
  * shared exponent s = floor(log2(max |x|)) - 2 (2 = the largest E2M1 exponent), clamped to
    [-127, 127]; s = -127 for an all-zero block; the scale byte is s + 127;
  * each element x / 2^s is rounded to the nearest E2M1 magnitude, ties to the even code
    (mantissa bit 0), and magnitudes past 6 go to 6 (the nearest value there); the sign bit is
    the sign of x, except that a zero magnitude is always code 0.
Element 2i of a row sits in the low nibble of byte i, element 2i + 1 in the high nibble.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E2M1_EMAX = 2


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code from its bit fields (subnormal when the exponent is 0)."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = (m / 2.0) if e == 0 else (2.0 ** (e - 1)) * (1.0 + m / 2.0)
    return -mag if s else mag


E2M1_MAGNITUDES = np.array([e2m1_value(c) for c in range(8)], dtype=np.float64)


def shared_exponent(block: np.ndarray) -> int:
    amax = float(np.max(np.abs(block)))
    if amax == 0.0:
        return -127
    _, e = np.frexp(amax)            # amax = f * 2^e, f in [0.5, 1): floor(log2(amax)) = e - 1
    return int(min(127, max(-127, (e - 1) - E2M1_EMAX)))


def round_e2m1(v: float) -> int:
    """Code (0..15) of the E2M1 value nearest to v, ties to the even code."""
    a = abs(v)
    d = np.abs(E2M1_MAGNITUDES - a)
    best = np.flatnonzero(d == d.min())
    c = int(best[0]) if best.size == 1 else int(best[(best & 1) == 0][0])
    if c == 0:
        return 0
    return c | (8 if v < 0 else 0)


def quantize(x) -> tuple[np.ndarray, np.ndarray]:
    """Codes (one uint8 per element, 0..15) and scale bytes of rows x[..., dim], dim % 32 == 0.

    The rounding of round_e2m1, for all elements at once: |x| / 2^s lies between two adjacent
    magnitudes, and the midpoints between neighbours are the decision points -- the count of
    midpoints below it is the nearest magnitude's code; a value on a midpoint is a tie and
    goes to the even code of the two."""
    x = np.asarray(x, dtype=np.float64)
    dim = x.shape[-1]
    assert dim % BLOCK == 0
    blocks = x.reshape(-1, BLOCK)
    codes = np.empty(blocks.shape, dtype=np.uint8)
    scales = np.empty(blocks.shape[0], dtype=np.uint8)
    mids = (E2M1_MAGNITUDES[:-1] + E2M1_MAGNITUDES[1:]) / 2     # 0.25, 0.75, ..., 5
    for i0 in range(0, blocks.shape[0], 1 << 16):      # bounded temporaries
        blk = blocks[i0:i0 + (1 << 16)]
        amax = np.abs(blk).max(axis=-1)
        _, e = np.frexp(amax)
        s = np.where(amax == 0.0, -127, np.clip((e - 1) - E2M1_EMAX, -127, 127)).astype(np.int64)
        y = blk * np.ldexp(1.0, -s)[:, None]           # exact: a power-of-two scaling
        a = np.abs(y)
        c = np.searchsorted(mids, a, side="left")       # midpoints strictly below a
        tie = (c < mids.size) & (a == mids[np.minimum(c, mids.size - 1)])
        c = np.where(tie & ((c & 1) == 1), c + 1, c)    # on a midpoint: the even code
        codes[i0:i0 + blk.shape[0]] = np.where((c != 0) & (y < 0), c | 8, c)
        scales[i0:i0 + blk.shape[0]] = s + 127
    return codes.reshape(x.shape), scales.reshape(x.shape[:-1] + (dim // BLOCK,))


def dequantize(codes, scales) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    dim = codes.shape[-1]
    vals = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
    v = np.take(vals, codes).reshape(codes.shape[:-1] + (dim // BLOCK, BLOCK))
    s = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return (v * s[..., None]).reshape(codes.shape)


def pack(codes) -> np.ndarray:
    """Two codes per byte: element 2i low nibble, 2i + 1 high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out
