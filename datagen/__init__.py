"""Seeded synthetic inputs for the CSA hot path.

This module draws random tensors and rounds them to the storage dtype. It holds
none of the method's arithmetic (no pooling, scoring, selection or attention):
both the HIP path and the float64 oracle consume exactly the tensors built here.

Seeds: every tensor is drawn from
``numpy.random.Generator(PCG64(SeedSequence([ROOT, case_id, tensor_id, attempt, *extra])))``
so a tensor can be redrawn alone (``attempt`` > 0) without touching the others.
Large tensors are drawn in fixed chunks of ``CHUNK`` values, chunk ``k`` using the
extra key ``k``; the result does not depend on how many threads draw them.

Shapes and distributions follow the five workloads of the CSA hot path (compressed
entries of dim 512 shared as key and value, 64x128 indexer, Top-512, window 128):
"DeepSeek V4-Flash: The Cost of Deciding What to Read", sections "Rebuilding the model
from its constants" (CSA layer table), "The Lightning Indexer", "The sliding window is
not an optimisation"; "DeepSeek-V4.1-Flash's KV-Cache Compression, Checked Down to the
Byte", section 3 (hierarchical pool of 2,048 blocks x 8 positions).
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

ROOT = 20261202
CHUNK = 1 << 22

# tensor ids (stable: changing one changes every stored seed)
T_X, T_Z, T_BIAS, T_XI, T_ZI, T_BIAS_I = 0, 1, 2, 3, 4, 5
T_KV, T_KI, T_Q, T_QI, T_W, T_SINK, T_QI2, T_W2 = 6, 7, 8, 9, 10, 11, 12, 13
T_QX, T_RINGX, T_SINKX, T_POS = 14, 15, 16, 17
T_XB, T_ZB, T_BIAS_B, T_XB_STALE = 18, 19, 20, 21


def _gen(case_id: int, tid: int, attempt: int = 0, *extra: int) -> np.random.Generator:
    ss = np.random.SeedSequence([ROOT, int(case_id), int(tid), int(attempt), *[int(e) for e in extra]])
    return np.random.Generator(np.random.PCG64(ss))


def normal(case_id: int, tid: int, shape, attempt: int = 0, *extra: int) -> np.ndarray:
    """Standard normal float32 array, drawn in CHUNK-sized pieces (threaded for big tensors)."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.float32)
    nchunk = max(1, (n + CHUNK - 1) // CHUNK)

    def fill(k: int) -> None:
        lo, hi = k * CHUNK, min(n, (k + 1) * CHUNK)
        if hi > lo:
            out[lo:hi] = _gen(case_id, tid, attempt, *extra, k).standard_normal(hi - lo, dtype=np.float32)

    if nchunk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(max_workers=min(16, nchunk)) as ex:
            list(ex.map(fill, range(nchunk)))
    return out.reshape(shape)


def to_storage(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Round an array to the storage dtype ('bf16' by round-to-nearest-even, or 'f32')."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t.clone()
    raise ValueError(dtype)


def lognormal_rows(case_id: int, tid: int, shape, sigma: float) -> np.ndarray:
    """Rows with uniformly random direction and log-normal norm exp(sigma * N(0,1))."""
    g = normal(case_id, tid, shape)
    rows = int(np.prod(shape[:-1]))
    r = np.exp(sigma * normal(case_id, tid, (rows,), 0, 1_000_003)).astype(np.float32)
    flat = g.reshape(rows, shape[-1])
    nrm = np.sqrt(np.einsum("ij,ij->i", flat, flat, dtype=np.float32))
    flat *= (r / np.maximum(nrm, 1e-30))[:, None]
    return flat.reshape(shape)


@dataclasses.dataclass
class CaseSpec:
    """One synthetic workload. ``kind`` is 'decode' (one new token per sequence, the fused
    decode step) or 'prefill' (a chunk of queries at the end of the context)."""
    case_id: int
    kind: str
    dtype: str = "bf16"
    B: int = 1                 # sequences
    L: int = 1024              # context length (tokens) including the new token / chunk
    m: int = 4                 # compression ratio
    H_I: int = 64
    d_I: int = 128
    H: int = 64
    D: int = 512
    K: int = 512
    W: int = 128
    w_cap: int = 128           # ring capacity (rows)
    e_cap: int | None = None   # cache capacity (entries); default L // m
    chunk: int = 0             # prefill: number of query tokens at the end of the context
    block_size: int = 0        # hierarchical pre-select (0 = off)
    max_blocks: int = 0
    n_attn: int = 1            # attention calls sharing one selection
    key_sigma: float = 0.0     # >0: log-normal key norms
    unit_scale: bool = True    # True: every tensor N(0,1)/sqrt(last dim) (sink N(0,1))
    bias_sigma: float | None = None
    ragged: bool = False       # decode: per-sequence positions differ
    scale: float | None = None
    compressor: str = "single"  # decode main entries: "single" stream or "c4a" (overlapped)

    @property
    def entries(self) -> int:
        return self.e_cap if self.e_cap is not None else self.L // self.m

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.D)


# The five workloads. Sizes per the workload descriptions; see the module docstring.
CONFIGS = {
    1: CaseSpec(1, "tiny", dtype="f32", B=1, L=2048, m=4, H_I=4, d_I=32, H=4, D=64, K=64, W=64,
                w_cap=2048, unit_scale=False, bias_sigma=0.1, scale=0.125),
    2: CaseSpec(2, "decode", B=8, L=65536, m=4, w_cap=128),
    3: CaseSpec(3, "prefill", B=1, L=131072, m=4, w_cap=8192, chunk=4096),
    4: CaseSpec(4, "decode", B=4, L=1048576, m=4, w_cap=128, key_sigma=0.5),
    5: CaseSpec(5, "decode", B=4, L=262144, m=1, w_cap=128, block_size=8, max_blocks=2048, n_attn=3),
}

# A second workload beyond the five: Heavily Compressed Attention at 1M context (m' = 128, one
# stream, no indexer: dense attention over every entry, 8,192 per sequence, plus the window).
HCA_DECODE = CaseSpec(6, "decode", B=4, L=1048576, m=128, K=8192, w_cap=128, key_sigma=0.5)

WORKLOAD_NAMES = {
    1: "tiny CSA forward fp32, 2048 tokens, 512 entries, 4x32 indexer, 4x64 heads",
    2: "decode bf16, batch 8, 65,536 ctx (16,384 entries)",
    3: "chunked prefill bf16, 4,096 queries at the end of 131,072 ctx (32,768 entries)",
    4: "1M-ctx decode bf16, batch 4, 1,048,576 ctx (262,144 entries), log-normal key norms",
    5: "hierarchical decode bf16, batch 4, 262,144 ctx 1:1, pool 2,048x8, 3 attention calls",
    6: "HCA decode bf16, batch 4, 1,048,576 ctx 128:1 (8,192 entries), dense attention",
}


def _u(spec: CaseSpec, tid: int, shape, dim: int, attempt: int = 0, *extra: int) -> np.ndarray:
    a = normal(spec.case_id, tid, shape, attempt, *extra)
    if spec.unit_scale:
        a *= np.float32(1.0 / math.sqrt(dim))
    return a


def _rows(spec: CaseSpec, tid: int, shape, dim: int) -> np.ndarray:
    if spec.key_sigma > 0:
        return lognormal_rows(spec.case_id, tid, shape, spec.key_sigma)
    return _u(spec, tid, shape, dim)


def ring_from_raw(spec: CaseSpec) -> bool:
    """Whether attention call 0's window rows are the raw main rows (the compressor input).
    True when entries pool m > 1 tokens; 1:1 workloads keep a separate local ring per call."""
    return spec.m > 1


def positions(spec: CaseSpec) -> np.ndarray:
    """Decode: the position of each sequence's new token. Ragged cases spread them over
    [L/2, L-1] with a seeded draw; otherwise every sequence sits at L-1."""
    if not spec.ragged:
        return np.full(spec.B, spec.L - 1, dtype=np.int64)
    g = _gen(spec.case_id, T_POS)
    t = g.integers(spec.L // 2, spec.L, size=spec.B, dtype=np.int64)
    t[0] = spec.L - 1
    return t


def make_decode(spec: CaseSpec) -> dict:
    """Inputs of one fused decode step (one new token per sequence).

    The state holds: compressed caches ``kv`` [B,E,D] and ``k_idx`` [B,E,d_I] with every
    entry before the current block filled; the compressor tails of the current block
    (``x_tail``/``z_tail`` main, ``xi_tail``/``zi_tail`` indexer, [B,m,*]); one window ring
    per attention call [B,w_cap,D] holding the rows of positions < t at row p % w_cap.
    Call 0's ring holds the raw main rows (the compressor input) unless the workload is
    1:1 (m == 1), where every call has its own local ring that already holds position t.
    """
    assert spec.kind == "decode"
    B, m, D, dI, E = spec.B, spec.m, spec.D, spec.d_I, spec.entries
    dt = spec.dtype
    t = positions(spec)
    out = {"spec": spec, "pos": torch.from_numpy(t.copy())}
    out["kv"] = to_storage(_rows(spec, T_KV, (B, E, D), D), dt)
    out["k_idx"] = to_storage(_rows(spec, T_KI, (B, E, dI), dI), dt)
    # raw rows of the last w_cap positions (main stream) and the indexer stream's last m rows
    raw = _u(spec, T_X, (B, spec.w_cap, D), D)          # raw[b, j] = position t_b - w_cap + 1 + j
    zr = _u(spec, T_Z, (B, m, D), D)                    # logits of the current block's rows
    xi = _u(spec, T_XI, (B, m, dI), dI)
    zi = _u(spec, T_ZI, (B, m, dI), dI)
    bias_scale = spec.bias_sigma
    bias = _u(spec, T_BIAS, (m, D), D)
    bias_i = _u(spec, T_BIAS_I, (m, dI), dI)
    if bias_scale is not None:
        bias = normal(spec.case_id, T_BIAS, (m, D)) * np.float32(bias_scale)
        bias_i = normal(spec.case_id, T_BIAS_I, (m, dI)) * np.float32(bias_scale)
    x_tail = np.zeros((B, m, D), np.float32)
    z_tail = np.zeros((B, m, D), np.float32)
    xi_tail = np.zeros((B, m, dI), np.float32)
    zi_tail = np.zeros((B, m, dI), np.float32)
    rings = np.zeros((spec.n_attn, B, spec.w_cap, D), np.float32)
    x_new = np.zeros((B, D), np.float32)
    for b in range(B):
        tb = int(t[b])
        slot = tb % m
        # current block's earlier rows: positions tb-slot .. tb-1, then the new row at tb
        for j in range(slot + 1):
            p = tb - slot + j
            src = spec.w_cap - 1 - (tb - p)
            x_tail[b, j] = raw[b, src]
            z_tail[b, j] = zr[b, j]
            xi_tail[b, j] = xi[b, j]
            zi_tail[b, j] = zi[b, j]
        x_new[b] = raw[b, spec.w_cap - 1]
        for j in range(spec.w_cap):
            p = tb - spec.w_cap + 1 + j
            if p < 0:
                continue
            rings[0, b, p % spec.w_cap] = raw[b, j]
    # Call 0's ring holds the raw main rows when entries pool several tokens; in 1:1
    # workloads (and for calls > 0) each call owns a local ring that already holds position t.
    first_own = 0 if not ring_from_raw(spec) else 1
    for c in range(first_own, spec.n_attn):
        rings[c] = _u(spec, T_RINGX, (B, spec.w_cap, D), D, 0, c)
    new_slots = np.array([int(tb) % m for tb in t])
    out["x_new"] = to_storage(x_new, dt)
    out["z_new"] = to_storage(z_tail[np.arange(B), new_slots], dt)
    out["xi_new"] = to_storage(xi_tail[np.arange(B), new_slots], dt)
    out["zi_new"] = to_storage(zi_tail[np.arange(B), new_slots], dt)
    # the tails as stored before the step: the new token's slot is stale (zero)
    for arr in (x_tail, z_tail, xi_tail, zi_tail):
        arr[np.arange(B), new_slots] = 0.0
    out["x_tail"] = to_storage(x_tail, dt)
    out["z_tail"] = to_storage(z_tail, dt)
    out["xi_tail"] = to_storage(xi_tail, dt)
    out["zi_tail"] = to_storage(zi_tail, dt)
    out["bias"] = to_storage(bias, dt)
    out["bias_i"] = to_storage(bias_i, dt)
    if ring_from_raw(spec):
        # call 0's ring does not yet hold the new row (the step writes it)
        for b in range(B):
            rings[0, b, int(t[b]) % spec.w_cap] = 0.0
    out["rings"] = [to_storage(rings[c], dt) for c in range(spec.n_attn)]
    if spec.compressor == "c4a":
        out.update(_c4a_state(spec, t))
    out["q_idx"] = to_storage(_u(spec, T_QI, (B, spec.H_I, dI), dI), dt)
    out["w"] = to_storage(_u(spec, T_W, (B, spec.H_I), spec.H_I), dt).float()
    if spec.block_size > 0:
        out["q_idx2"] = to_storage(_u(spec, T_QI2, (B, spec.H_I, dI), dI), dt)
        out["w2"] = to_storage(_u(spec, T_W2, (B, spec.H_I), spec.H_I), dt).float()
    qs, sinks = [], []
    for c in range(spec.n_attn):
        tid_q = T_Q if c == 0 else T_QX
        qs.append(to_storage(_u(spec, tid_q, (B, spec.H, D), D, 0, c), dt))
        s = normal(spec.case_id, T_SINK if c == 0 else T_SINKX, (spec.H,), 0, c)
        sinks.append(to_storage(s, dt).float())
    out["q"] = qs
    out["sink"] = sinks
    out["scale"] = spec.softmax_scale
    return out


def _c4a_state(spec: CaseSpec, t: np.ndarray) -> dict:
    """The second (b) stream of the overlapped main compressor: its rows and logits for the
    new token (``xb_new``/``zb_new`` [B,D]), its positional bias ``bias_b`` [m,D], and the
    b rows of the last two blocks (``xb_tail``/``zb_tail`` [B,2m,D], position p at row
    p % 2m: the previous block whole, the current block up to t - 1). Rows of positions
    < 0 are zero; the rows the current block has not reached yet (positions t .. of its
    slots) hold stale values from an older block, drawn at random, never zero."""
    B, m, D, dt = spec.B, spec.m, spec.D, spec.dtype
    xb = _u(spec, T_XB, (B, 2 * m, D), D)     # xb[b, j] = position (block start - m + j)
    zb = _u(spec, T_ZB, (B, 2 * m, D), D)
    stale_x = _u(spec, T_XB_STALE, (B, 2 * m, D), D)
    stale_z = _u(spec, T_XB_STALE, (B, 2 * m, D), D, 1)
    if spec.bias_sigma is not None:
        bias_b = normal(spec.case_id, T_BIAS_B, (m, D)) * np.float32(spec.bias_sigma)
    else:
        bias_b = _u(spec, T_BIAS_B, (m, D), D)
    xb_tail, zb_tail = stale_x.copy(), stale_z.copy()
    xb_new = np.zeros((B, D), np.float32)
    zb_new = np.zeros((B, D), np.float32)
    for b in range(B):
        tb = int(t[b])
        s0 = tb - tb % m
        for j in range(m + tb % m):           # positions s0 - m .. tb - 1
            p = s0 - m + j
            xb_tail[b, p % (2 * m)] = xb[b, j] if p >= 0 else 0.0
            zb_tail[b, p % (2 * m)] = zb[b, j] if p >= 0 else 0.0
        xb_new[b] = xb[b, m + tb % m]
        zb_new[b] = zb[b, m + tb % m]
    return {"xb_new": to_storage(xb_new, dt), "zb_new": to_storage(zb_new, dt),
            "xb_tail": to_storage(xb_tail, dt), "zb_tail": to_storage(zb_tail, dt),
            "bias_b": to_storage(bias_b, dt), "compressor": "c4a"}


def redraw_w(spec: CaseSpec, which: str, b: int, attempt: int, dtype: str | None = None) -> torch.Tensor:
    """A fresh gate vector for sequence/query row ``b`` (``which`` = 'w' or 'w2')."""
    tid = T_W if which == "w" else T_W2
    a = normal(spec.case_id, tid, (spec.H_I,), attempt, b)
    if spec.unit_scale:
        a *= np.float32(1.0 / math.sqrt(spec.H_I))
    return to_storage(a, dtype or spec.dtype).float()


def redraw_qw(spec: CaseSpec, b: int, attempt: int) -> tuple[torch.Tensor, torch.Tensor]:
    """Fresh (q_idx row, gate row) for query row ``b`` (tiny workload: with 4 heads a gate
    redraw alone cannot split an exact tie of all-zero scores)."""
    q = normal(spec.case_id, T_QI, (spec.H_I, spec.d_I), attempt, b)
    w = normal(spec.case_id, T_W, (spec.H_I,), attempt, b)
    if spec.unit_scale:
        q *= np.float32(1.0 / math.sqrt(spec.d_I))
        w *= np.float32(1.0 / math.sqrt(spec.H_I))
    return to_storage(q, spec.dtype), to_storage(w, spec.dtype).float()


def make_prefill(spec: CaseSpec) -> dict:
    """Inputs of a chunked prefill: ``chunk`` query tokens at positions [L-chunk, L).

    Entries before the chunk are pre-filled in ``kv``/``k_idx``; the chunk's own entries
    come from compressing its raw rows (``x_chunk``/``z_chunk`` main, ``xi_chunk``/``zi_chunk``
    indexer), written by the caller into the caches at entry (L-chunk)/m. The ring holds the
    raw main rows of positions [L-chunk-W+1, L) at row p % w_cap.
    """
    B, m, D, dI, E, C = spec.B, spec.m, spec.D, spec.d_I, spec.entries, spec.chunk
    assert spec.kind in ("prefill", "tiny") and C % m == 0 and spec.L % m == 0
    # the ring holds positions [L-C-W+1, L) at row p % w_cap: they must not wrap onto each other
    assert spec.w_cap >= C + spec.W - 1, "ring capacity below chunk + window - 1"
    dt = spec.dtype
    L = spec.L
    t0 = L - C
    e0 = t0 // m
    out = {"spec": spec}
    kv = _rows(spec, T_KV, (B, E, D), D)
    ki = _rows(spec, T_KI, (B, E, dI), dI)
    kv[:, e0:] = 0.0
    ki[:, e0:] = 0.0
    out["kv"] = to_storage(kv, dt)
    out["k_idx"] = to_storage(ki, dt)
    n_raw = C + spec.W - 1
    raw = _u(spec, T_X, (B, n_raw, D), D)           # positions [t0-W+1, L)
    out["x_chunk"] = to_storage(raw[:, spec.W - 1:], dt)
    out["z_chunk"] = to_storage(_u(spec, T_Z, (B, C, D), D), dt)
    out["xi_chunk"] = to_storage(_u(spec, T_XI, (B, C, dI), dI), dt)
    out["zi_chunk"] = to_storage(_u(spec, T_ZI, (B, C, dI), dI), dt)
    out["bias"] = to_storage(_u(spec, T_BIAS, (m, D), D), dt)
    out["bias_i"] = to_storage(_u(spec, T_BIAS_I, (m, dI), dI), dt)
    ring = np.zeros((B, spec.w_cap, D), np.float32)
    for j in range(n_raw):
        p = t0 - spec.W + 1 + j
        if p >= 0:
            ring[:, p % spec.w_cap] = raw[:, j]
    out["ring"] = to_storage(ring, dt)
    out["q_pos"] = torch.arange(t0, L, dtype=torch.int64).repeat(B, 1)
    out["e_count"] = torch.full((B,), E, dtype=torch.int32)
    out["q_idx"] = to_storage(_u(spec, T_QI, (B, C, spec.H_I, dI), dI), dt)
    out["w"] = to_storage(_u(spec, T_W, (B, C, spec.H_I), spec.H_I), dt).float()
    out["q"] = to_storage(_u(spec, T_Q, (B, C, spec.H, D), D), dt)
    out["sink"] = to_storage(normal(spec.case_id, T_SINK, (spec.H,)), dt).float()
    out["scale"] = spec.softmax_scale
    return out


def make_prefill_indexer(spec: CaseSpec) -> dict:
    """The indexer's share of ``make_prefill``'s inputs, drawn identically (same seeds, same
    values): the indexer cache ``k_idx`` (the chunk's entries zero, to be pooled from
    ``xi_chunk``/``zi_chunk`` with ``bias_i``), ``q_idx``, ``w``, ``q_pos`` and ``e_count``."""
    B, m, dI, E, C = spec.B, spec.m, spec.d_I, spec.entries, spec.chunk
    assert spec.kind == "prefill" and C % m == 0 and spec.L % m == 0
    dt = spec.dtype
    e0 = (spec.L - C) // m
    ki = _rows(spec, T_KI, (B, E, dI), dI)
    ki[:, e0:] = 0.0
    out = {"spec": spec, "k_idx": to_storage(ki, dt)}
    out["xi_chunk"] = to_storage(_u(spec, T_XI, (B, C, dI), dI), dt)
    out["zi_chunk"] = to_storage(_u(spec, T_ZI, (B, C, dI), dI), dt)
    out["bias_i"] = to_storage(_u(spec, T_BIAS_I, (m, dI), dI), dt)
    out["q_pos"] = torch.arange(spec.L - C, spec.L, dtype=torch.int64).repeat(B, 1)
    out["e_count"] = torch.full((B,), E, dtype=torch.int32)
    out["q_idx"] = to_storage(_u(spec, T_QI, (B, C, spec.H_I, dI), dI), dt)
    out["w"] = to_storage(_u(spec, T_W, (B, C, spec.H_I), spec.H_I), dt).float()
    return out


def make_tiny(spec: CaseSpec) -> dict:
    """The tiny fp32 forward: one sequence of L tokens, all L queries. Raw rows X double as
    the window rows (ring capacity L); the indexer keys are given per entry."""
    B, m, D, dI, L = spec.B, spec.m, spec.D, spec.d_I, spec.L
    E = L // m
    dt = spec.dtype
    out = {"spec": spec}
    out["x"] = to_storage(normal(spec.case_id, T_X, (B, L, D)), dt)
    out["z"] = to_storage(normal(spec.case_id, T_Z, (B, L, D)), dt)
    out["bias"] = to_storage(normal(spec.case_id, T_BIAS, (m, D)) * np.float32(spec.bias_sigma or 1.0), dt)
    out["k_idx"] = to_storage(normal(spec.case_id, T_KI, (B, E, dI)), dt)
    out["q_idx"] = to_storage(normal(spec.case_id, T_QI, (B, L, spec.H_I, dI)), dt)
    out["w"] = to_storage(normal(spec.case_id, T_W, (B, L, spec.H_I)), dt).float()
    out["q"] = to_storage(normal(spec.case_id, T_Q, (B, L, spec.H, D)), dt)
    out["sink"] = to_storage(normal(spec.case_id, T_SINK, (spec.H,)), dt).float()
    out["q_pos"] = torch.arange(L, dtype=torch.int64).repeat(B, 1)
    out["e_count"] = torch.full((B,), E, dtype=torch.int32)
    out["scale"] = spec.softmax_scale
    return out


def make_case(spec: CaseSpec) -> dict:
    if spec.kind == "decode":
        return make_decode(spec)
    if spec.kind == "prefill":
        return make_prefill(spec)
    if spec.kind == "tiny":
        return make_tiny(spec)
    raise ValueError(spec.kind)


def tensor(case_id: int, tid: int, shape, dtype: str = "bf16", scale: float = 1.0,
           attempt: int = 0, *extra: int) -> torch.Tensor:
    """An ad-hoc seeded tensor: N(0,1) * scale rounded to the storage dtype."""
    a = normal(case_id, tid, shape, attempt, *extra)
    if scale != 1.0:
        a *= np.float32(scale)
    return to_storage(a, dtype)
