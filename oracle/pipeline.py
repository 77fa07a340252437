"""Row-by-row oracle drivers for the library calls -- TEST INFRASTRUCTURE ONLY.

Each driver loops over sequences and queries and applies the float64 primitives of
``oracle.csa`` in the order the pages describe: compress -> visibility -> index score
-> Top-K (or block pre-select -> pool rescoring -> Top-K) -> sparse attention with sink.
Inputs may be torch CPU tensors or NumPy arrays; they are upcast exactly to float64.
Sources as in ``oracle.csa``.
"""
from __future__ import annotations

import numpy as np

from . import csa, fp8, kv_fp4, mx


def f64(a) -> np.ndarray:
    """Exact upcast of a bf16/fp32 torch tensor or array to a float64 NumPy array."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return a.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(a, dtype=np.float64)


def i64(a) -> np.ndarray:
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return a.detach().to("cpu").to(torch.int64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(a, dtype=np.int64)


def take_rows(a, ids) -> np.ndarray:
    """Rows ``a[ids]`` of a torch tensor or array, upcast exactly to float64."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return f64(a[torch.as_tensor(np.asarray(ids, dtype=np.int64))])
    except ImportError:  # pragma: no cover
        pass
    return f64(np.asarray(a)[np.asarray(ids, dtype=np.int64)])


def compress(x, z, bias, m: int, dtype: str) -> np.ndarray:
    """csa_compress: pooled entries rounded to the storage dtype."""
    return csa.store(csa.compress(f64(x), f64(z), f64(bias), m), dtype)


def index_topk_row(q_idx, w, k_idx, t: int, m: int, e_count: int, K: int, cand=None):
    """One query row of csa_index_topk. Returns (ids ascending -1 padded, float64 scores of
    the scored candidates, candidate ids scored)."""
    n = csa.n_visible(t, m, e_count)
    if cand is None:
        ids = np.arange(n, dtype=np.int64)
    else:
        c = i64(cand)
        ids = c[(c >= 0) & (c < n)]
    keys = f64(k_idx)[ids] if ids.size else np.zeros((0, np.asarray(k_idx).shape[-1]))
    s = csa.index_scores(f64(q_idx), f64(w), keys) if ids.size else np.zeros(0)
    return csa.select_topk(s, K, index=ids), s, ids


def index_topk(q_idx, w, k_idx, q_pos, e_count, m: int, K: int, rows=None, cand=None):
    """csa_index_topk over (sequence, query) rows. q_idx [B,Q,H_I,d_I], w [B,Q,H_I],
    k_idx [B,E,d_I], q_pos [B,Q], e_count [B] or None, cand [B,Q,n_cand] or None.
    ``rows``: optional list of (b, i) to evaluate (default all). Returns dict (b,i) -> ids."""
    qp = i64(q_pos)
    B, Q = qp.shape
    E = k_idx.shape[1]
    ec = i64(e_count) if e_count is not None else np.full(B, E)
    rows = rows if rows is not None else [(b, i) for b in range(B) for i in range(Q)]
    res = {}
    keys_cache = {}
    for b, i in rows:
        if b not in keys_cache:
            keys_cache = {b: f64(k_idx[b])}
        c = None if cand is None else cand[b, i]
        res[(b, i)] = index_topk_row(q_idx[b, i], w[b, i], keys_cache[b], int(qp[b, i]), m,
                                     int(min(ec[b], E)), K, cand=c)
    return res


def index_blocks_row(q_idx, w, k_idx, t: int, m: int, e_count: int, block_size: int,
                     max_blocks: int):
    """One query row of csa_index_blocks: the candidate pool (ascending ids) and the
    stage-1 scores of the visible entries."""
    n = csa.n_visible(t, m, e_count)
    keys = f64(k_idx)[:n]
    s = csa.index_scores(f64(q_idx), f64(w), keys)
    return csa.candidate_pool(s, block_size, max_blocks), s


def attend_row(q, kv, idx, ring, w_cap: int, window: int, t: int, sink, scale: float):
    """One query row of csa_sparse_attn (float64, unrounded)."""
    rows = csa.attention_rows(kv, idx, ring, w_cap, window, t)
    return csa.sink_attention(f64(q), rows, None if sink is None else f64(sink), scale)


def sparse_attn(q, kv, idx, ring, w_cap, window, q_pos, sink, scale, dtype, rows=None):
    """csa_sparse_attn over rows (b, i); returns dict (b, i) -> stored output [H, D]."""
    qp = i64(q_pos)
    B, Q = qp.shape
    idx = i64(idx)
    rows = rows if rows is not None else [(b, i) for b in range(B) for i in range(Q)]
    out = {}
    for b, i in rows:
        sel = idx[b, i]
        sel = sel[sel >= 0]
        kvr = np.zeros((0, kv.shape[-1])) if sel.size == 0 else take_rows(kv[b], sel)
        # attention_rows indexes kv by id: pass the gathered rows with local ids
        o = attend_row(q[b, i], kvr, np.arange(sel.size), f64(ring[b]), w_cap, window,
                       int(qp[b, i]), sink, scale)
        out[(b, i)] = csa.store(o, dtype)
    return out


def cached_index_key(case: dict, key) -> np.ndarray:
    """The indexer key of a new entry as the cache holds it: the pooled key in the step's
    dtype, then, for an MXFP4 cache (case["idx_format"] "mxfp4" or "mxfp4_qk"), its MXFP4
    value ("FP4, down to the index scores": the indexer's keys are cached in FP4)."""
    if case.get("idx_format") in ("mxfp4", "mxfp4_qk"):
        return mx.dequantize(*mx.quantize(key))
    return key


def index_query(case: dict, q) -> np.ndarray:
    """The indexer query [heads, dim] the scores multiply: as given, or, on the FP4 query-key
    path (case["idx_format"] == "mxfp4_qk"), each head's MXFP4 value under the keys' rule
    ([CoD] "FP4, down to the index scores": the indexer's query-key path is cached, loaded and
    multiplied entirely in FP4; the products of two FP4 values are exact)."""
    q = f64(q)
    if case.get("idx_format") == "mxfp4_qk":
        return mx.dequantize(*mx.quantize(q))
    return q


def prepare_kv_row(case: dict, v, t: int) -> np.ndarray:
    """A key/value row of the shared-KV attention as the step stores it, unrounded: the
    per-head RMSNorm with case["kv_gamma"] (when given), then RoPE at position t on the last
    case["kv_rope_dim"] channels (when > 0).

    [CoD "Key and value are the same vector": RMSNorm per head on the single KV head just
    before the core attention; RoPE on the last 64 dimensions, so a cached row carries the
    rotation of its position and the inverse rotation of the output at -t leaves each row's
    contribution a function of its distance from the query.] [CoD, vLLM's serving notes
    in "Two cache hierarchies, and lcm(4, 128)": KV RoPE is fused with the sliding-window key
    insertion.] Reading: a window row is a key/value row of the same attention as a pooled
    entry, so it is prepared the same way, at its own position; t is the newest token the
    row holds (the pooled entry's last position, the window row's own position)."""
    v = f64(v)
    if case.get("kv_gamma") is not None:
        v = csa.rms_norm(v[None], f64(case["kv_gamma"]), 1e-6)[0]
    if case.get("kv_rope_dim"):
        v = csa.rope(v[None], float(t), int(case["kv_rope_dim"]))[0]
    return v


def kv_row_prepared(case: dict) -> bool:
    """Whether the step normalises or rotates the key/value rows it stores."""
    return case.get("kv_gamma") is not None or bool(case.get("kv_rope_dim"))


def cached_main_entry(v, kv_format):
    """The value a main cache in kv_format ("fp8", "fp4", or None for the path's dtype) holds
    for an entry v already rounded to that dtype."""
    if kv_format == "fp8":
        return fp8.cached_entries(v)
    if kv_format == "fp4":
        return kv_fp4.cached_entries(v)
    return v


def decode_step(case: dict, seqs=None) -> dict:
    """The fused decode step for one new token per sequence (oracle side).

    Per sequence b at position t: the new rows enter the compressor tails at slot t % m
    (and call 0's ring at row t % w_cap when its window rows are the raw main rows); if
    the block is complete ((t+1) % m == 0) entry (t+1)/m - 1 is pooled from the tails for
    both streams and stored; then the visible entries are scored, selected (directly, or
    through the block pre-select and pool rescoring), and every attention call attends to
    the shared selection plus its own window and sink. With case["idx_format"] == "mxfp4",
    case["k_idx"] holds the MXFP4 values of the cached keys and the new entry's key is
    quantised before it is scored (``cached_index_key``); "mxfp4_qk" quantises the indexer
    query to MXFP4 as well (``index_query``). With case["score_format"] == "bf16"
    the flat selection ranks the scores rounded fp64 -> fp32 -> bf16. With
    case["out_rope_dim"] > 0 every output head's last channels are turned back by RoPE at -t
    ([CoD] "Key and value are the same vector") before the store; case["q_gamma"] (per call, or
    None) and case["q_rope_dim"] prepare each call's query (RMSNorm, RoPE at +t) first. With
    case["kv_format"] == "fp8" (or "fp4"), case["kv"] holds the values of an FP8 main cache
    (576-byte entries, oracle/fp8.py; or 288-byte FP4 entries, oracle/kv_fp4.py) and the new
    entry is attended at its cached value. case["kv_gamma"]
    and case["kv_rope_dim"] give the new entry its per-head RMSNorm and RoPE (at t, the position
    of the newest token it pools) before it is stored (rounded once), and the new window row
    the same at its position t (``prepare_kv_row``). With case["compressor"] == "c4a" the main
    entry is the overlapped two-stream pooling ([CoD] "The compressor has two streams and they
    overlap"): the new b-stream row enters case["xb_tail"] (the b rows of the last two blocks,
    position p at row p % 2m) and entry e pools the a rows of its own block with the b rows of
    block e - 1 (none for e = 0) through ``csa.compress_c4a``; the indexer keys keep the
    single-stream pooling.
    Returns a dict with per-sequence results (new entries, scores, pool, ids, outputs).
    """
    spec = case["spec"]
    m, dt, E, K, W, wc = spec.m, spec.dtype, spec.entries, spec.K, spec.W, spec.w_cap
    pos = i64(case["pos"])
    seqs = list(range(spec.B)) if seqs is None else list(seqs)
    ring_raw = spec.m > 1
    c4a = case.get("compressor") == "c4a"
    res = {"ids": {}, "out": {}, "kv_new": {}, "kv_new_exact": {}, "ki_new": {}, "scores": {},
           "pool": {}, "win_row": {}, "win_row_exact": {},
           "scores2": {}, "n_vis": {}}
    bias, bias_i = f64(case["bias"]), f64(case["bias_i"])
    for b in seqs:
        t = int(pos[b])
        slot = t % m
        x_tail = f64(case["x_tail"][b]).copy()
        z_tail = f64(case["z_tail"][b]).copy()
        xi_tail = f64(case["xi_tail"][b]).copy()
        zi_tail = f64(case["zi_tail"][b]).copy()
        x_tail[slot] = f64(case["x_new"][b])
        z_tail[slot] = f64(case["z_new"][b])
        xi_tail[slot] = f64(case["xi_new"][b])
        zi_tail[slot] = f64(case["zi_new"][b])
        if c4a:
            xb_ring = f64(case["xb_tail"][b]).copy()
            zb_ring = f64(case["zb_tail"][b]).copy()
            xb_ring[t % (2 * m)] = f64(case["xb_new"][b])
            zb_ring[t % (2 * m)] = f64(case["zb_new"][b])
        n_vis = csa.n_visible(t, m, E)
        keys = f64(case["k_idx"][b][:n_vis]).copy()
        new_e = None
        if (t + 1) % m == 0:
            new_e = (t + 1) // m - 1
            # the new entry's single head: RMSNorm, then RoPE at the position of the newest
            # token it pools (t)
            if c4a:
                # a rows: this block (the tail); b rows: block new_e - 1, the other half of
                # the two-block ring, absent for the sequence's first entry
                prev_x = prev_z = None
                if new_e > 0:
                    h = ((new_e - 1) % 2) * m
                    prev_x, prev_z = xb_ring[h:h + m], zb_ring[h:h + m]
                pooled = csa.compress_c4a(x_tail, z_tail, np.zeros_like(x_tail),
                                          np.zeros_like(z_tail), bias, f64(case["bias_b"]), m,
                                          Xb_prev=prev_x, Zb_prev=prev_z)[0]
            else:
                pooled = csa.compress(x_tail, z_tail, bias, m)[0]
            kv_p = prepare_kv_row(case, pooled, t)
            kv_e = csa.store(kv_p, dt)
            res["kv_new_exact"][b] = kv_p
            ki_e = csa.store(csa.compress(xi_tail, zi_tail, bias_i, m)[0], dt)
            res["kv_new"][b] = kv_e
            res["ki_new"][b] = ki_e
            if new_e < n_vis:
                keys[new_e] = cached_index_key(case, ki_e)
        res["n_vis"][b] = n_vis
        s1 = csa.index_scores(index_query(case, case["q_idx"][b]), f64(case["w"][b]), keys)
        if case.get("score_format") == "bf16":
            # the fp32 scores quantised to BF16 ahead of the selection ([CoD] "FP4, down to
            # the index scores"); ties at the K-th value go to the lower id as before
            s1 = csa.round_bf16(csa.round_f32(s1))
        res["scores"][b] = s1
        if spec.block_size > 0:
            pool = csa.candidate_pool(s1, spec.block_size, spec.max_blocks)
            s2 = csa.index_scores(f64(case["q_idx2"][b]), f64(case["w2"][b]), keys[pool])
            ids = csa.select_topk(s2, K, index=pool)
            res["pool"][b] = pool
            res["scores2"][b] = s2
        else:
            ids = csa.select_topk(s1, K)
        res["ids"][b] = ids
        sel = ids[ids >= 0]
        kv_rows = take_rows(case["kv"][b], sel) if sel.size else np.zeros((0, spec.D))
        if new_e is not None:
            kv_rows[sel == new_e] = cached_main_entry(res["kv_new"][b], case.get("kv_format"))
        outs = []
        for c in range(spec.n_attn):
            ring = f64(case["rings"][c][b]).copy()
            if c == 0 and ring_raw:
                # the new raw row enters the window prepared like an entry, at its position t
                xw = f64(case["x_new"][b])
                if kv_row_prepared(case):
                    res["win_row_exact"][b] = prepare_kv_row(case, xw, t)
                    xw = csa.store(res["win_row_exact"][b], dt)
                ring[t % wc] = xw
                res["win_row"][b] = xw
            q = case["q"][c][b]
            qg = (case.get("q_gamma") or [None] * spec.n_attn)[c]
            qr = int(case.get("q_rope_dim", 0))
            if qg is not None or qr:
                # the query's per-head RMSNorm and RoPE at +t, stored at the step's precision
                q = f64(q)
                if qg is not None:
                    q = csa.rms_norm(q, f64(qg), 1e-6)
                if qr:
                    q = csa.rope(q, float(t), qr)
                q = csa.store(q, dt)
            o = attend_row(q, kv_rows, np.arange(sel.size), ring, wc, W, t,
                           case["sink"][c], case["scale"])
            if case.get("out_rope_dim"):
                # RoPE at -t on the last out_rope_dim channels of each head's output
                o = csa.rope(o, -float(t), int(case["out_rope_dim"]))
            outs.append(csa.store(o, dt))
        res["out"][b] = outs
    return res


def prefill_entries(case: dict):
    """Entries of a prefill chunk: pooled main entries and indexer keys (stored dtype)."""
    spec = case["spec"]
    kv_c = compress(case["x_chunk"], case["z_chunk"], case["bias"], spec.m, spec.dtype)
    ki_c = compress(case["xi_chunk"], case["zi_chunk"], case["bias_i"], spec.m, spec.dtype)
    return kv_c, ki_c


def prefill_rows(case: dict, rows, kv_c=None, ki_c=None) -> dict:
    """Chunked prefill, oracle side, for query rows (b, i): ids and stored outputs."""
    spec = case["spec"]
    if kv_c is None:
        kv_c, ki_c = prefill_entries(case)
    e0 = (spec.L - spec.chunk) // spec.m
    qp = i64(case["q_pos"])
    res = {"ids": {}, "out": {}, "scores": {}}
    cache = {}
    for b, i in rows:
        if b not in cache:
            kv = f64(case["kv"][b]).copy()
            ki = f64(case["k_idx"][b]).copy()
            kv[e0:e0 + kv_c.shape[1]] = kv_c[b]
            ki[e0:e0 + ki_c.shape[1]] = ki_c[b]
            cache = {b: (kv, ki)}
        kv, ki = cache[b]
        t = int(qp[b, i])
        ids, s, _ = index_topk_row(case["q_idx"][b, i], case["w"][b, i], ki, t, spec.m,
                                   spec.entries, spec.K)
        o = attend_row(case["q"][b, i], kv, ids, f64(case["ring"][b]), spec.w_cap, spec.W, t,
                       case["sink"], case["scale"])
        res["ids"][(b, i)] = ids
        res["scores"][(b, i)] = s
        res["out"][(b, i)] = csa.store(o, spec.dtype)
    return res


def tiny_forward(case: dict, rows=None) -> dict:
    """The tiny fp32 forward: compress the raw rows, then every query row (b, t) indexes,
    selects and attends (window rows read from the raw rows themselves)."""
    spec = case["spec"]
    kv = compress(case["x"], case["z"], case["bias"], spec.m, spec.dtype)
    qp = i64(case["q_pos"])
    B, Q = qp.shape
    rows = rows if rows is not None else [(b, i) for b in range(B) for i in range(Q)]
    res = {"kv": kv, "ids": {}, "out": {}, "scores": {}}
    for b, i in rows:
        t = int(qp[b, i])
        ids, s, _ = index_topk_row(case["q_idx"][b, i], case["w"][b, i], f64(case["k_idx"][b]),
                                   t, spec.m, kv.shape[1], spec.K)
        o = attend_row(case["q"][b, i], kv[b], ids, f64(case["x"][b]), spec.L, spec.W, t,
                       case["sink"], case["scale"])
        res["ids"][(b, i)] = ids
        res["scores"][(b, i)] = s
        res["out"][(b, i)] = csa.store(o, spec.dtype)
    return res
