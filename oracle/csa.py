"""Float64 CPU oracle for the CSA hot path -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import, call or run anything in this package. The product path (libcsa and its
Python binding) never does, and this package imports nothing from it.

Every function computes the plain definition of one step, in float64, on the exact
values handed to the GPU (bf16 inputs upcast exactly). Tensors the method *stores*
(compressed entries, attention outputs) are rounded to the storage dtype at the point
of storage; index scores are rounded to fp32 before selection because the pages take
the Top-K decision on FP32 index scores.

Sources (page titles; sections named as on the page):
  [CoD]  "DeepSeek V4-Flash: The Cost of Deciding What to Read" (The Software Frontier)
  [B890] "DeepSeek-V4.1-Flash's KV-Cache Compression, Checked Down to the Byte" (flozi-tech)
  [V41]  "DeepSeek-V4.1-Flash" interactive architecture study (shuhuayu.github.io)

Readings taken where the pages are silent or garbled (each is listed with its reason in
the design notes): half-open entry ranges; the positional bias is added to the logits;
non-overlapping single-stream pooling; window rows = raw rows ending at the query
(inclusive); no deduplication between window and selected rows; no scale on the index
score; Top-K output ascending with -1 padding and ties to the lower index; blocks of the
hierarchical pre-select aligned to entry 0, only visible entries counted.

Parity pins: every function here is pinned by the CPU tests under tests/ (closed forms,
library routines, invariants, brute force and hand-worked fixtures in tests/golden/).
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------------------
# storage rounding
# ----------------------------------------------------------------------------------------


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even (returned as float64).

    bfloat16 keeps 8 significant bits and float32's exponent range: a normal value
    mant * 2**exp (0.5 <= |mant| < 1) has quantum 2**(exp - 8); below 2**-126 the quantum
    stays 2**-133 (subnormals). Magnitudes that round to 2**128 or beyond become inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0.0)
    xf = x[fin]
    _, e = np.frexp(xf)
    eq = np.maximum(e, -125) - 8
    q = np.rint(np.ldexp(xf, -eq))          # rint: round half to even
    r = np.ldexp(q, eq)
    r[np.abs(r) >= 2.0 ** 128] = np.copysign(np.inf, xf[np.abs(r) >= 2.0 ** 128])
    out[fin] = r
    return out


def round_f32(x) -> np.ndarray:
    """Round float64 values to float32 (IEEE round to nearest even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def store(x, dtype: str) -> np.ndarray:
    """Round a computed float64 tensor to the storage dtype ('bf16' or 'f32')."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------------------
# a1: compressor -- learned channel-wise softmax pooling
# ----------------------------------------------------------------------------------------


def compress(X, Z, bias, m: int) -> np.ndarray:
    """Pool every m consecutive rows into one compressed entry, channel by channel.

    [CoD "The compressor has two streams and they overlap": the compression weights are
    per dimension and a softmax over the pooled positions runs independently for each
    channel; the entry is the weighted sum of the pooled rows.]
    [CoD "Rebuilding the model from its constants", CSA/HCA layer tables: a learnable
    positional bias of shape m x 512 per stream; HCA pools with one stream.]
    [V41 "CSA2: separate producing, selecting, and reading": a learned channel-wise softmax
    pools each group; groups do not overlap.]

    X, Z: [..., T, d] raw rows and their compression logits; bias: [m, d]; T % m == 0.
    Entry e covers positions [e*m, (e+1)*m). For channel c:
        a_j   = Z[e*m + j, c] + bias[j, c]                (j = position within the entry)
        alpha = softmax_j(a)
        out[e, c] = sum_j alpha_j * X[e*m + j, c]
    Returns float64 [..., T/m, d] (unrounded).
    """
    X = np.asarray(X, dtype=np.float64)
    Z = np.asarray(Z, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    T, d = X.shape[-2], X.shape[-1]
    if T % m != 0:
        raise ValueError("token count must be a multiple of m")
    if bias.shape != (m, d):
        raise ValueError("bias must be [m, d]")
    E = T // m
    lead = X.shape[:-2]
    Xb = X.reshape(lead + (E, m, d))
    A = Z.reshape(lead + (E, m, d)) + bias            # bias indexed by position within entry
    A = A - A.max(axis=-2, keepdims=True)
    P = np.exp(A)
    P /= P.sum(axis=-2, keepdims=True)                # softmax over the m positions, per channel
    return (P * Xb).sum(axis=-2)


def compress_c4a(Xa, Za, Xb, Zb, bias_a, bias_b, m: int, Xb_prev=None, Zb_prev=None) -> np.ndarray:
    """The overlapped two-stream compressor (vLLM's "c4a" at m = 4).

    [CoD "The compressor has two streams and they overlap": two independent projections C^a
    and C^b with their own compression logits Z^a and Z^b; entry i takes C^a from positions
    [m i, m(i+1)) and C^b from [m(i-1), m i) (the page prints closed brackets; half-open as in
    the single-stream reading), a softmax over the concatenated 2m logits per channel and a
    weighted sum over both streams -- eight tokens at stride four for m = 4.]
    [CoD "Rebuilding the model from its constants", CSA layer table: positional biases B^a,
    B^b of shape m x 512, one per stream.]

    Xa, Za, Xb, Zb: [..., T, d] rows of positions p0 .. p0 + T - 1 (p0 a multiple of m), T % m
    == 0; bias_a, bias_b: [m, d]. Xb_prev, Zb_prev: [..., m, d] the b-stream rows of the m
    positions before p0, or None when p0 = 0 -- entry 0 of a sequence has no b-part (reading:
    positions before the sequence are masked, so its softmax runs over its m a-logits only).
    For chunk entry e and channel c, with lists over j < m:
        logits  = [Za[m e + j] + bias_a[j]] + [Zb[m(e-1) + j] + bias_b[j]]   (b-part: the
                  previous block, from Xb_prev/Zb_prev for e = 0)
        alpha   = softmax over all of them
        out[e]  = sum of alpha times the matching rows Xa[m e + j] and Xb[m(e-1) + j]
    Returns float64 [..., T/m, d] (unrounded).
    """
    Xa, Za, Xb, Zb = (np.asarray(t, dtype=np.float64) for t in (Xa, Za, Xb, Zb))
    ba, bb = np.asarray(bias_a, dtype=np.float64), np.asarray(bias_b, dtype=np.float64)
    T, d = Xa.shape[-2], Xa.shape[-1]
    if T % m != 0:
        raise ValueError("token count must be a multiple of m")
    E = T // m
    lead = Xa.shape[:-2]
    if (Xb_prev is None) != (Zb_prev is None):
        raise ValueError("give both previous b-stream blocks or neither")
    out = np.empty(lead + (E, d))
    for e in range(E):
        la = Za[..., m * e:m * e + m, :] + ba                    # [..., m, d]
        xa = Xa[..., m * e:m * e + m, :]
        if e > 0:
            lb = Zb[..., m * (e - 1):m * e, :] + bb
            xb = Xb[..., m * (e - 1):m * e, :]
        elif Xb_prev is not None:
            lb = np.asarray(Zb_prev, dtype=np.float64) + bb
            xb = np.asarray(Xb_prev, dtype=np.float64)
        else:
            lb = xb = None
        L = la if lb is None else np.concatenate([la, lb], axis=-2)
        X = xa if xb is None else np.concatenate([xa, xb], axis=-2)
        P = np.exp(L - L.max(axis=-2, keepdims=True))
        P /= P.sum(axis=-2, keepdims=True)                      # softmax over 2m (or m)
        out[..., e, :] = (P * X).sum(axis=-2)
    return out


def rms_norm(x, gamma, eps: float = 1e-6) -> np.ndarray:
    """Per-vector RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gamma.

    [CoD "Key and value are the same vector" (the output-projection passage): RMSNorm per head
    on the queries and on the single head of the compressed KV entries, just before the core
    attention; the norm weights are learned.] eps is not printed on the pages:
    1e-6 (reading)."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope(x, pos, rope_dim: int = 64, base: float = 10000.0) -> np.ndarray:
    """Rotary position embedding on the last rope_dim channels of each vector.

    [CoD "Key and value are the same vector": RoPE on the last 64 dimensions of each head;
    applying it with position -i to the output undoes a rotation R(i) because R is orthogonal
    and R(t)^-1 R(s) = R(s-t).] Not printed on the pages (reading): channel pairs (2j, 2j+1)
    of the rotated part, angle pos * base^(-2j/rope_dim), base 10000 -- the original RoPE form.
    x [..., d]; pos broadcastable to x[..., 0] (per vector). Returns float64."""
    x = np.asarray(x, dtype=np.float64).copy()
    d = x.shape[-1]
    p = np.asarray(pos, dtype=np.float64)[..., None]
    j = np.arange(rope_dim // 2, dtype=np.float64)
    ang = p * base ** (-2.0 * j / rope_dim)
    c, s_ = np.cos(ang), np.sin(ang)
    a = x[..., d - rope_dim::2].copy()
    b = x[..., d - rope_dim + 1::2].copy()
    x[..., d - rope_dim::2] = a * c - b * s_
    x[..., d - rope_dim + 1::2] = a * s_ + b * c
    return x


# ----------------------------------------------------------------------------------------
# causal visibility of compressed entries
# ----------------------------------------------------------------------------------------


def n_visible(t: int, m: int, e_count: int | None = None) -> int:
    """Number of compressed entries a query at position t may read.

    [CoD "The sliding window is not an optimisation": an entry summarising positions
    m*i .. m*(i+1)-1 is usable by a query at t only if m*(i+1)-1 <= t.] So entries
    0 .. floor((t+1)/m)-1 are visible, further capped by the entries actually present.
    """
    if t < 0:
        return 0
    n = (int(t) + 1) // int(m)
    if e_count is not None:
        n = min(n, int(e_count))
    return n


# ----------------------------------------------------------------------------------------
# a2: lightning-indexer score
# ----------------------------------------------------------------------------------------


def index_scores(q_idx, w, k_idx) -> np.ndarray:
    """I(t, s) = sum_h w(t,h) * ReLU(q_I(t,h) . K_s) for one query over keys k_idx.

    [CoD "The Lightning Indexer": 64 indexer heads of dim 128, one compressed indexer key per
    entry, a rectified dot product per head, summed across heads with a per-head gate w.
    No scale factor appears in the score.]

    q_idx [H_I, d_I], w [H_I], k_idx [n, d_I] -> float64 [n].
    """
    return head_relu(q_idx, k_idx) @ np.asarray(w, dtype=np.float64)


def head_relu(q_idx, k_idx) -> np.ndarray:
    """R[s, h] = ReLU(q_I(t,h) . K_s): the per-head rectified dot products of one query
    before the gate-weighted head sum. q_idx [H_I, d_I], k_idx [n, d_I] -> float64 [n, H_I]."""
    q = np.asarray(q_idx, dtype=np.float64)
    k = np.asarray(k_idx, dtype=np.float64)
    return np.maximum(k @ q.T, 0.0)


def score_scale(q_idx, w, k_idx) -> np.ndarray:
    """A(t, s) = sum_h |w(t,h)| * ReLU(q_I(t,h) . K_s): the natural error scale of a score
    (the same sum with every term's magnitude). Used by tolerances, not by the method."""
    q = np.asarray(q_idx, dtype=np.float64)
    w = np.abs(np.asarray(w, dtype=np.float64))
    k = np.asarray(k_idx, dtype=np.float64)
    return np.maximum(k @ q.T, 0.0) @ w


# ----------------------------------------------------------------------------------------
# a3: Top-K selection
# ----------------------------------------------------------------------------------------


def select_topk(scores, K: int, index=None) -> np.ndarray:
    """Keep the K highest-scoring candidates; ties go to the lower index.

    [CoD "The Lightning Indexer": a cheap scoring pass picks the top 512 and attention runs
    only over those; Flash's top-k is 512.] [CoD "FP4, down to the index scores": the index
    scores are FP32 (BF16 only as a further optimisation), so the decision is taken on the
    fp32-rounded score.]

    scores [n] (float64; rounded to fp32 here), index [n] the global id of each candidate
    (default 0..n-1). Returns int64 [K]: the selected ids in ascending order, -1 padded
    when fewer than K candidates exist.
    """
    s = round_f32(np.asarray(scores, dtype=np.float64))
    n = s.shape[0]
    idx = np.arange(n, dtype=np.int64) if index is None else np.asarray(index, dtype=np.int64)
    out = np.full(K, -1, dtype=np.int64)
    if n == 0 or K == 0:
        return out
    # lexsort: last key is primary -> descending score (-0.0 == +0.0), then ascending id
    order = np.lexsort((idx, -s))
    chosen = np.sort(idx[order[: min(K, n)]])
    out[: chosen.shape[0]] = chosen
    return out


# ----------------------------------------------------------------------------------------
# a4: hierarchical pre-select (block maxima -> candidate pool)
# ----------------------------------------------------------------------------------------


def block_maxima(scores, block_size: int) -> np.ndarray:
    """Bmax[b] = max of the (fp32) scores of the visible entries in block b, where block b
    covers entries [b*bs, (b+1)*bs). [V41 "Hierarchical indexing bounds the deeper
    searches": each 8-position block is scored by its maximum.] scores covers exactly the
    visible entries, so the last block may be partial."""
    s = round_f32(np.asarray(scores, dtype=np.float64))
    n = s.shape[0]
    nb = (n + block_size - 1) // block_size
    out = np.empty(nb, dtype=np.float64)
    for b in range(nb):
        out[b] = s[b * block_size: min(n, (b + 1) * block_size)].max()
    return out


def candidate_pool(scores, block_size: int, max_blocks: int) -> np.ndarray:
    """Entries of the max_blocks blocks with the highest maxima, ascending.

    [B890 section 3: the first Full layer scores the whole visible range and does blockwise
    candidate selection, at most 2,048 blocks of 8 positions, a pool of up to 16,384
    candidates.] [V41 "Hierarchical indexing bounds the deeper searches".]
    Blocks are ranked by (maximum desc, block id asc); blocks with no visible entry do not
    exist here. Returns int64 ids of the pool's (visible) entries in ascending order.
    """
    bm = block_maxima(scores, block_size)
    blocks = select_topk(bm, max_blocks)
    n = np.asarray(scores).shape[0]
    parts = [np.arange(b * block_size, min(n, (b + 1) * block_size), dtype=np.int64)
             for b in blocks if b >= 0]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


# ----------------------------------------------------------------------------------------
# a5: sparse attention over selected entries + window, with a per-head sink
# ----------------------------------------------------------------------------------------


def attention_rows(kv, idx, ring, w_cap: int, window: int, t: int):
    """The rows a query at position t attends to, in order: the selected compressed
    entries (ids in idx, -1 skipped), then the raw window rows of positions
    max(0, t-window+1) .. t, read from ring row p % w_cap.

    [CoD "The sliding window is not an optimisation": 128 uncompressed tokens are
    concatenated with the selected entries before the softmax.] [B890 section 5: a query
    at position i attends to window keys in [max(s, i-W+1), i].] [CoD "Key and value are
    the same vector": each row serves as both key and value.]
    """
    kv = np.asarray(kv, dtype=np.float64)
    ring = np.asarray(ring, dtype=np.float64)
    sel = [int(i) for i in np.asarray(idx).ravel() if int(i) >= 0]
    rows = [kv[i] for i in sel]
    if window > 0 and t >= 0:
        for p in range(max(0, t - window + 1), t + 1):
            rows.append(ring[p % w_cap])
    if not rows:
        return np.zeros((0, kv.shape[-1]), dtype=np.float64)
    return np.stack(rows)


def sink_attention(q, rows, sink, scale: float) -> np.ndarray:
    """Softmax attention of every head over ``rows`` (keys = values), with a per-head sink.

    [CoD "Attention sink, and heads that abstain": for head h, exp(z'_h) is added to the
    softmax denominator and to nothing else:
        s(h,i,j) = exp(z(h,i,j)) / (sum_k exp(z(h,i,k)) + exp(z'_h)) ]
    z(h, j) = scale * q_h . row_j. q [H, D], rows [J, D], sink [H] (None: no sink).
    Returns float64 [H, D]; zero when there are no rows.
    """
    q = np.asarray(q, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    H, D = q.shape
    if rows.shape[0] == 0:
        return np.zeros((H, D), dtype=np.float64)
    z = scale * (q @ rows.T)                          # [H, J]
    M = z.max(axis=1)
    if sink is not None:
        sink = np.asarray(sink, dtype=np.float64)
        M = np.maximum(M, sink)
    p = np.exp(z - M[:, None])
    den = p.sum(axis=1)
    if sink is not None:
        den = den + np.exp(sink - M)
    return (p @ rows) / den[:, None]
