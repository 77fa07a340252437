"""Algorithmic work of the CSA hot path: bytes and FLOPs the method itself must move or
compute, used for roofline fractions. Over-fetch, score round-trips and repeated reads
earn no credit; dense work the method avoids is never counted.

Sources: "DeepSeek V4-Flash: The Cost of Deciding What to Read", sections "The Lightning
Indexer" and "The indexer is O(n), and that is the ceiling" (the indexer scans every visible
entry; the selector is ~79% of attention FLOPs at 1M and half at 32K);
"DeepSeek-V4.1-Flash's KV-Cache Compression, Checked Down to the Byte", section 3
(indexer MACs = heads x dim x positions; pool of 2,048 blocks x 8).
"""
from __future__ import annotations

import dataclasses
import math

BF16 = 2
F32 = 4


def indexer_macs(heads: int, dim: int, positions: int) -> int:
    """Multiply-accumulates of one query's indexer scan over ``positions`` keys."""
    return heads * dim * positions


def selector_share(ctx: int, n_csa: int = 21, n_hca: int = 20, n_swa: int = 2, heads: int = 64,
                   head_dim: int = 512, idx_heads: int = 64, idx_dim: int = 128, m: int = 4,
                   m_hca: int = 128, top_k: int = 512, window: int = 128) -> float:
    """Fraction of a decode token's attention MACs spent in the CSA indexer scan.

    Per query and layer: indexer idx_heads*idx_dim*floor(ctx/m); CSA core attention
    2*heads*head_dim*(min(top_k, ctx/m) + window) (scores and weighted sum over shared
    key=value rows); HCA 2*heads*head_dim*(ceil(ctx/m_hca) + window); SWA
    2*heads*head_dim*window. The page prints the resulting share (79% at 1M, half at 32K)
    without its formula; this is the plainest accounting that uses only the page's dims.
    """
    e = ctx // m
    idx = indexer_macs(idx_heads, idx_dim, e)
    core = 2 * heads * head_dim * (min(top_k, e) + window)
    hca = 2 * heads * head_dim * (math.ceil(ctx / m_hca) + window)
    swa = 2 * heads * head_dim * window
    total = n_csa * (idx + core) + n_hca * hca + n_swa * swa
    return n_csa * idx / total


@dataclasses.dataclass
class StepBytes:
    keys: int          # indexer keys of the scanned entries (stage 1 + pool)
    gather: int        # selected + window rows read by attention
    queries: int       # q, q_idx (+ second query), gates, sinks
    outputs: int       # attention outputs and selected ids
    compress: int      # tails + new rows read, new entries + ring row written

    @property
    def total(self) -> int:
        return self.keys + self.gather + self.queries + self.outputs + self.compress


def decode_step_bytes(B: int, n_vis: int, m: int, D: int, H: int, H_I: int, d_I: int, K: int,
                      W: int, n_attn: int = 1, pool: int = 0, elt: int = BF16,
                      ring_write: bool = True, key_bytes: int | None = None,
                      entry_bytes: int | None = None, c4a: bool = False) -> StepBytes:
    """Algorithmic HBM bytes of one fused decode step over B sequences, each with n_vis
    visible entries (all sequences at a block boundary, so one entry is pooled per stream).
    pool > 0: hierarchical (stage-1 scan of n_vis keys, then ``pool`` rescored keys).
    key_bytes: bytes of one cached indexer key (default d_I * elt; MXFP4: mxfp4_key_bytes).
    entry_bytes: bytes of one cached main entry (default D * elt; FP8: FP8_ENTRY_BYTES; FP4:
    FP4_ENTRY_BYTES).
    c4a: the overlapped main compressor adds its b stream: the new b row (x and z) read and
    written to its ring, the previous block's m b rows read, and its bias."""
    kb = d_I * elt if key_bytes is None else key_bytes
    eb = D * elt if entry_bytes is None else entry_bytes
    keys = B * n_vis * kb + B * pool * kb
    sel = min(K, pool if pool else n_vis)
    gather = n_attn * B * (sel * eb + W * D * elt)
    queries = B * (H_I * d_I * elt + H_I * F32) * (2 if pool else 1) + n_attn * B * H * D * elt \
        + n_attn * H * F32
    outputs = n_attn * B * H * D * elt + B * K * 4
    # compressor: m tail rows + the new row for both streams (x, z, xi, zi) read, the new
    # row written to the tails, one entry per stream written, the ring row written
    per_row = (2 * D + 2 * d_I) * elt
    compress = B * (m * per_row + per_row + eb + kb + (D * elt if ring_write else 0)) \
        + m * (D + d_I) * elt
    if c4a:
        compress += B * (2 * D * elt * (m + 2)) + m * D * elt
    return StepBytes(keys, gather, queries, outputs, compress)


# "What the cache costs, checked four ways": 64 bf16 rotary dims + 448 FP8 dims per entry
FP8_ENTRY_BYTES = 64 * 2 + 448
# "DeepSeek-V4.1-Flash's KV-Cache Compression, Checked Down to the Byte", section 4: 512 E2M1
# elements + one E4M3 scale byte per 16 channels
FP4_ENTRY_BYTES = 512 // 2 + 512 // 16


def mxfp4_key_bytes(d_I: int) -> int:
    """Bytes of one MXFP4 indexer key: a 4-bit code per channel and one scale byte per 32
    channels ("What the cache costs, checked four ways": 64 bytes of codes per 128-channel key)."""
    return d_I // 2 + d_I // 32


def scan_bytes(rows: int, n_keys: int, H_I: int, d_I: int, elt: int = BF16,
               key_bytes: int | None = None) -> int:
    """Algorithmic bytes of one indexer-scan launch: the keys of every scanned entry (d_I * elt
    each, or key_bytes) plus each row's query and gate (scores are an intermediate and earn
    nothing)."""
    kb = d_I * elt if key_bytes is None else key_bytes
    return rows * (n_keys * kb + H_I * d_I * elt + H_I * F32)


def prefill_indexer_flops(sum_visible: int, H_I: int, d_I: int) -> int:
    """FLOPs of the prefill indexer contraction over visible (query, entry) pairs only."""
    return 2 * H_I * d_I * sum_visible


def sum_visible(t0: int, t1: int, m: int, e_cap: int) -> int:
    """sum over t in [t0, t1) of min(e_cap, floor((t+1)/m))."""
    return sum(min(e_cap, (t + 1) // m) for t in range(t0, t1))
