"""Composition pins of the oracle's drivers (oracle/pipeline.py).

The drivers compose the pinned primitives into the results every GPU parity test compares
against: the chunked prefill, the tiny forward, the sparse-attention call, the block
pre-select, the candidate-list index call and the decode step's query preparation and output
inverse RoPE. Each test here rebuilds a driver's result in a loop of its own, straight from
the definitions on the pages:

  - index score, brute force per (query, key): sum_h w_h * max(0, q_h . k)
    ([CoD] "The Lightning Indexer");
  - Top-K by a full sort on (fp32 score desc, id asc), ids ascending, -1 padded;
  - attention per head with an explicit softmax whose denominator carries e^{sink}
    ([CoD] "Attention sink, and heads that abstain"), over the selected rows followed by the
    window rows of positions max(0, t-W+1) .. t ([CoD] "The sliding window is not an
    optimisation");
  - RoPE as a complex rotation of each channel pair, RMSNorm from the vector's L2 norm
    ([CoD] "Key and value are the same vector").

Each test also plants a plausible mistake in that independent composition (a wrong splice
offset, raw rows in place of pooled entries, a window shifted by one, -1 ids read as the last
row, blocks ranked by their sum, ...) and checks that the mistaken result falls outside the
same tolerance: the comparison can tell them apart.
"""
import cmath
import dataclasses
import math

import numpy as np
import pytest
import torch

import datagen
from oracle import csa, gaps, pipeline
from oracle.pipeline import f64

# ---------------------------------------------------------------------------------------
# brute-force definitions (no oracle arithmetic)
# ---------------------------------------------------------------------------------------


def bf_score(q, w, key) -> float:
    tot = 0.0
    for h in range(q.shape[0]):
        d = 0.0
        for c in range(q.shape[1]):
            d += float(q[h, c]) * float(key[c])
        tot += float(w[h]) * max(d, 0.0)
    return tot


def bf_topk(pairs, K: int) -> list:
    """pairs: (score, id). The K best by (fp32 score desc, id asc); ids ascending, -1 pad."""
    order = sorted(pairs, key=lambda p: (-float(np.float32(p[0])), p[1]))
    chosen = sorted(int(i) for _, i in order[:K])
    return chosen + [-1] * (K - len(chosen))


def bf_attend(q, rows, sink, scale: float) -> np.ndarray:
    H, D = q.shape
    out = np.zeros((H, D))
    for h in range(H):
        z = [scale * float(np.dot(q[h], r)) for r in rows]
        zs = None if sink is None else float(sink[h])
        cands = z + ([zs] if zs is not None else [])
        if not cands:
            continue
        M = max(cands)
        num = np.zeros(D)
        den = 0.0
        for zj, r in zip(z, rows):
            e = math.exp(zj - M)
            num += e * np.asarray(r, dtype=np.float64)
            den += e
        if zs is not None:
            den += math.exp(zs - M)
        if rows:
            out[h] = num / den
    return out


def bf_rope(v, p: float, rd: int, base: float = 10000.0) -> np.ndarray:
    v = np.array(v, dtype=np.float64)
    d = v.shape[-1]
    for j in range(rd // 2):
        a = d - rd + 2 * j
        z = complex(v[a], v[a + 1]) * cmath.exp(1j * p * base ** (-2.0 * j / rd))
        v[a], v[a + 1] = z.real, z.imag
    return v


def bf_rms(v, g, eps: float = 1e-6) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    return v * np.asarray(g, dtype=np.float64) * math.sqrt(v.size) / math.sqrt(
        float(np.dot(v, v)) + v.size * eps)


def store(x, dt):
    return csa.round_bf16(x) if dt == "bf16" else csa.round_f32(x)


def within(stored, exact, dt) -> bool:
    """A stored value matches the exact one: within a rounding step of the storage dtype
    (2^-8 relative for bf16, 2^-23 for fp32) plus 1e-12 of the largest magnitude (float64
    summation order)."""
    stored, exact = np.asarray(stored, dtype=np.float64), np.asarray(exact, dtype=np.float64)
    rel = 2.0 ** -8 if dt == "bf16" else 2.0 ** -23
    bound = rel * np.abs(exact) + 1e-12 * max(1.0, float(np.abs(exact).max(initial=0.0)))
    return bool(np.all(np.abs(stored - exact) <= bound))


# ---------------------------------------------------------------------------------------
# chunked prefill
# ---------------------------------------------------------------------------------------

PREFILL = datagen.CaseSpec(911, "prefill", B=1, L=512, m=4, H_I=8, d_I=16, H=4, D=32, K=16,
                           W=8, w_cap=128, chunk=64)
PREFILL_ROWS = [(0, 0), (0, 3), (0, 17), (0, 42), (0, 63)]


def bf_prefill_row(case, i, kv_c, ki_c, mistake=None):
    spec = case["spec"]
    m, L, C, W, wc = spec.m, spec.L, spec.chunk, spec.W, spec.w_cap
    t0 = L - C
    e0 = t0 // m + (1 if mistake == "e0" else 0)
    n_c = kv_c.shape[1]
    kv_pre, ki_pre = f64(case["kv"][0]), f64(case["k_idx"][0])
    # the caches with the chunk's entries spliced in at e0, built by concatenation
    kv = np.concatenate([kv_pre[:e0], kv_c[0], kv_pre[e0 + n_c:]])[:spec.entries]
    ki = np.concatenate([ki_pre[:e0], ki_c[0], ki_pre[e0 + n_c:]])[:spec.entries]
    t = t0 + i
    n = min((t + 1) // m, spec.entries)
    q_i, w_i = f64(case["q_idx"][0, i]), f64(case["w"][0, i])
    ids = bf_topk([(bf_score(q_i, w_i, ki[s]), s) for s in range(n)], spec.K)
    rows = [kv[s] for s in ids if s >= 0]
    ring, xc = f64(case["ring"][0]), f64(case["x_chunk"][0])
    for p in range(max(0, t - W + 1), t + 1):
        if mistake == "ring":
            rows.append(ring[(p + 1) % wc])
        else:
            # the chunk's own raw rows from x_chunk, earlier positions from the ring
            rows.append(xc[p - t0] if p >= t0 else ring[p % wc])
    o = bf_attend(f64(case["q"][0, i]), rows, f64(case["sink"]), case["scale"])
    return ids, o


def test_prefill_rows_match_brute_force_composition():
    case = datagen.make_case(PREFILL)
    gaps.enforce_prefill(case, PREFILL_ROWS)
    kv_c, ki_c = pipeline.prefill_entries(case)
    res = pipeline.prefill_rows(case, PREFILL_ROWS, kv_c, ki_c)
    t0 = PREFILL.L - PREFILL.chunk
    e0 = t0 // PREFILL.m
    saw_chunk_entry = False
    for (b, i) in PREFILL_ROWS:
        ids, o = bf_prefill_row(case, i, kv_c, ki_c)
        assert res["ids"][(b, i)].tolist() == ids
        assert within(res["out"][(b, i)], o, "bf16")
        saw_chunk_entry |= any(s >= e0 for s in ids)
    assert saw_chunk_entry                    # the chunk's spliced entries are selected
    # planted mistakes fail the same comparison on some row
    for mistake in ("e0", "ring"):
        bad = False
        for (b, i) in PREFILL_ROWS:
            ids, o = bf_prefill_row(case, i, kv_c, ki_c, mistake)
            bad |= res["ids"][(b, i)].tolist() != ids or not within(res["out"][(b, i)], o, "bf16")
        assert bad, mistake


def test_prefill_entries_are_the_pooled_chunk():
    case = datagen.make_case(PREFILL)
    kv_c, ki_c = pipeline.prefill_entries(case)
    m = PREFILL.m
    x, z, bias = f64(case["x_chunk"][0]), f64(case["z_chunk"][0]), f64(case["bias"])
    for e in (0, 7, 15):
        # entry e pools chunk rows m e .. m e + m - 1 by a per-channel softmax with the bias
        for c in (0, 5, 31):
            a = [z[m * e + j, c] + bias[j, c] for j in range(m)]
            mx = max(a)
            wts = [math.exp(v - mx) for v in a]
            want = sum(wt * x[m * e + j, c] for j, wt in enumerate(wts)) / sum(wts)
            assert abs(kv_c[0, e, c] - want) <= 2.0 ** -8 * abs(want) + 1e-12


def test_prefill_ring_must_hold_the_chunk_and_window():
    # positions [L-chunk-W+1, L) must fit the ring without wrapping onto themselves
    with pytest.raises(AssertionError):
        datagen.make_case(dataclasses.replace(PREFILL, w_cap=64))


# ---------------------------------------------------------------------------------------
# tiny forward
# ---------------------------------------------------------------------------------------

TINY = datagen.CaseSpec(912, "tiny", dtype="f32", B=1, L=256, m=4, H_I=4, d_I=32, H=4, D=64,
                        K=16, W=16, w_cap=256, unit_scale=False, bias_sigma=0.1, scale=0.125)
TINY_ROWS = [(0, 0), (0, 9), (0, 35), (0, 70), (0, 255)]   # n_vis 0, 2, 9, 17 > K, 64


def bf_tiny_row(case, t, mistake=None):
    spec = case["spec"]
    m, W = spec.m, spec.W
    x = f64(case["x"][0])
    # the entries: csa.compress of the raw rows (pinned by the compressor tests), fp32 stored
    kv = store(csa.compress(x, f64(case["z"][0]), f64(case["bias"]), m), "f32")
    ki = f64(case["k_idx"][0])
    n = (t + 1) // m
    q_i, w_i = f64(case["q_idx"][0, t]), f64(case["w"][0, t])
    ids = bf_topk([(bf_score(q_i, w_i, ki[s]), s) for s in range(n)], spec.K)
    if mistake == "raw":
        rows = [x[m * s + m - 1] for s in ids if s >= 0]
    else:
        rows = [kv[s] for s in ids if s >= 0]
    lo, hi = (t - W, t - 1) if mistake == "window" else (t - W + 1, t)
    rows += [x[p] for p in range(max(0, lo), hi + 1)]
    return ids, bf_attend(f64(case["q"][0, t]), rows, f64(case["sink"]), case["scale"])


def test_tiny_forward_matches_brute_force_composition():
    case = datagen.make_case(TINY)
    gaps.enforce_tiny(case)
    res = pipeline.tiny_forward(case, rows=TINY_ROWS)
    for (b, t) in TINY_ROWS:
        ids, o = bf_tiny_row(case, t)
        assert res["ids"][(b, t)].tolist() == ids
        assert within(res["out"][(b, t)], o, "f32")
    assert (res["ids"][(0, 70)] >= 0).sum() == 16 and (res["ids"][(0, 35)] >= 0).sum() == 9
    for mistake in ("raw", "window"):
        bad = any(not within(res["out"][r], bf_tiny_row(case, r[1], mistake)[1], "f32")
                  for r in TINY_ROWS[1:])
        assert bad, mistake


# ---------------------------------------------------------------------------------------
# sparse attention call over supplied ids
# ---------------------------------------------------------------------------------------


def test_sparse_attn_matches_brute_force_over_explicit_ids():
    B, Q, H, D, E, wc, W = 2, 3, 4, 32, 40, 16, 6
    kv = datagen.tensor(913, 0, (B, E, D), "bf16", 0.2)
    ring = datagen.tensor(913, 1, (B, wc, D), "bf16", 0.2)
    q = datagen.tensor(913, 2, (B, Q, H, D), "bf16", 1.0)
    sink = datagen.tensor(913, 3, (H,), "f32")
    rng = np.random.default_rng(913)
    K = 7
    idx = np.full((B, Q, K), -1, dtype=np.int64)
    for b in range(B):
        for i in range(Q):
            k = [3, 7, 0][i]                      # row 2: ids all -1 (window only)
            idx[b, i, :k] = rng.choice(E, size=k, replace=False)
            rng.shuffle(idx[b, i])                # any order, -1 anywhere
    q_pos = torch.tensor([[2, 9, 30], [5, 15, 39]], dtype=torch.int64)
    scale = 1.0 / math.sqrt(D)
    res = pipeline.sparse_attn(q, kv, torch.from_numpy(idx), ring, wc, W, q_pos, sink, scale,
                               "bf16")

    def brute(b, i, mistake=None):
        t = int(q_pos[b, i])
        kvb, rb = f64(kv[b]), f64(ring[b])
        if mistake == "neg":
            rows = [kvb[s] for s in idx[b, i]]      # -1 read as the last row
        else:
            rows = [kvb[s] for s in idx[b, i] if s >= 0]
        lo = t - W + 1 if mistake != "clamp" else t - W + 1 - 2
        rows += [rb[p % wc] for p in range(max(0, lo), t + 1)]
        return bf_attend(f64(q[b, i]), rows, f64(sink), scale)

    for b in range(B):
        for i in range(Q):
            assert within(res[(b, i)], brute(b, i), "bf16")
    for mistake in ("neg", "clamp"):
        assert any(not within(res[(b, i)], brute(b, i, mistake), "bf16")
                   for b in range(B) for i in range(Q)), mistake


# ---------------------------------------------------------------------------------------
# block pre-select (csa_index_blocks) and the candidate-list branch of csa_index_topk
# ---------------------------------------------------------------------------------------


def test_index_blocks_row_matches_brute_force():
    H_I, d_I, E, bs, mb, m = 4, 8, 53, 4, 5, 2
    q = f64(datagen.tensor(914, 0, (H_I, d_I), "bf16"))
    w = f64(datagen.tensor(914, 1, (H_I,), "bf16"))
    k = f64(datagen.tensor(914, 2, (E, d_I), "bf16"))

    def brute(t, rank="max"):
        n = min((t + 1) // m, E)
        s = [bf_score(q, w, k[e]) for e in range(n)]
        nb = (n + bs - 1) // bs
        blocks = []
        for blk in range(nb):
            vals = [float(np.float32(v)) for v in s[blk * bs:min(n, blk * bs + bs)]]
            blocks.append((max(vals) if rank == "max" else sum(vals), blk))
        keep = sorted(blocks, key=lambda p: (-p[0], p[1]))[:mb]
        pool = sorted(e for _, blk in keep for e in range(blk * bs, min(n, blk * bs + bs)))
        return pool, s

    for t in (0, 1, 8, 30, 70, 105, 200):          # partial last blocks, n < bs * mb, n = E
        pool, s = pipeline.index_blocks_row(q, w, k, t, m, E, bs, mb)
        want, s_bf = brute(t)
        assert pool.tolist() == want, t
        np.testing.assert_allclose(s, s_bf, rtol=1e-12, atol=1e-12)
    assert any(pipeline.index_blocks_row(q, w, k, t, m, E, bs, mb)[0].tolist() != brute(t, "sum")[0]
               for t in (30, 70, 105, 200))


def test_index_topk_candidate_list_matches_brute_force():
    H_I, d_I, E, m, K = 4, 8, 60, 4, 6
    q = f64(datagen.tensor(915, 0, (H_I, d_I), "bf16"))
    w = f64(datagen.tensor(915, 1, (H_I,), "bf16"))
    k = f64(datagen.tensor(915, 2, (E, d_I), "bf16"))
    cand = np.array([-1, 0, 2, 3, 9, 11, 12, 20, 31, 33, 41, 47, 55, 59, -1, -1])
    for t in (3, 50, 130, 239):
        n = min((t + 1) // m, E)
        ids, s, scored = pipeline.index_topk_row(q, w, k, t, m, E, K, cand=cand)
        ok = [int(c) for c in cand if 0 <= c < n]
        assert scored.tolist() == ok                          # -1 and ids past n_vis dropped
        want = bf_topk([(bf_score(q, w, k[c]), c) for c in ok], K)
        assert ids.tolist() == want, t
        # planted mistake: keeping the ids past the visible count
        leaky = bf_topk([(bf_score(q, w, k[c]), c) for c in cand if c >= 0], K)
        if n < 59:
            assert leaky != want or all(c < n for c in leaky)


# ---------------------------------------------------------------------------------------
# decode step: query preparation, entry and window-row preparation, output inverse RoPE
# ---------------------------------------------------------------------------------------


def prepared_case(dt="bf16", **kw):
    base = dict(case_id=916, kind="decode", dtype=dt, B=2, L=1024, m=4, H_I=8, d_I=16, H=4,
                D=32, K=8, W=8, w_cap=16, ragged=True)
    base.update(kw)
    case = datagen.make_case(datagen.CaseSpec(**base))
    D = case["spec"].D
    tt = torch.float32 if dt == "f32" else torch.bfloat16
    case["q_gamma"] = [datagen.tensor(916, 40, (D,), dt, 0.3).abs().to(tt) + 0.5]
    case["kv_gamma"] = datagen.tensor(916, 41, (D,), dt, 0.3).abs().to(tt) + 0.5
    case["q_rope_dim"] = 16
    case["kv_rope_dim"] = 16
    case["out_rope_dim"] = 16
    return case


def bf_decode_seq(case, b, mistake=None):
    spec = case["spec"]
    m, D, W, wc, dt = spec.m, spec.D, spec.W, spec.w_cap, spec.dtype
    t = int(case["pos"][b])
    rd, qrd, ord_ = case["kv_rope_dim"], case["q_rope_dim"], case["out_rope_dim"]
    g_kv, g_q = f64(case["kv_gamma"]), f64(case["q_gamma"][0])
    kv = {e: f64(case["kv"][b][e]) for e in range(spec.entries)}
    ki = {e: f64(case["k_idx"][b][e]) for e in range(spec.entries)}
    if (t + 1) % m == 0:
        e = (t + 1) // m - 1
        xt, zt = f64(case["x_tail"][b]).copy(), f64(case["z_tail"][b]).copy()
        xit, zit = f64(case["xi_tail"][b]).copy(), f64(case["zi_tail"][b]).copy()
        xt[t % m], zt[t % m] = f64(case["x_new"][b]), f64(case["z_new"][b])
        xit[t % m], zit[t % m] = f64(case["xi_new"][b]), f64(case["zi_new"][b])
        pooled = csa.compress(xt, zt, f64(case["bias"]), m)[0]
        kv[e] = store(bf_rope(bf_rms(pooled, g_kv), t, rd), dt)
        ki[e] = store(csa.compress(xit, zit, f64(case["bias_i"]), m)[0], dt)
    n = min((t + 1) // m, spec.entries)
    q_i, w_i = f64(case["q_idx"][b]), f64(case["w"][b])
    ids = bf_topk([(bf_score(q_i, w_i, ki[s]), s) for s in range(n)], spec.K)
    rows = [kv[s] for s in ids if s >= 0]
    ring = f64(case["rings"][0][b])
    x_new = f64(case["x_new"][b])
    for p in range(max(0, t - W + 1), t + 1):
        if p == t:
            rows.append(x_new if mistake == "raw_window" else
                        store(bf_rope(bf_rms(x_new, g_kv), t, rd), dt))
        else:
            rows.append(ring[p % wc])
    qv = np.stack([bf_rms(v, g_q) for v in f64(case["q"][0][b])])
    if mistake != "no_qrope":
        qv = np.stack([bf_rope(v, t, qrd) for v in qv])
    qv = store(qv, dt)
    o = bf_attend(qv, rows, f64(case["sink"][0]), case["scale"])
    sign = 1.0 if mistake == "out_sign" else -1.0
    o = np.stack([bf_rope(v, sign * t, ord_) for v in o])
    return ids, o


def test_decode_step_preparation_matches_brute_force():
    case = prepared_case()
    gaps.enforce_decode(case)
    spec = case["spec"]
    res = pipeline.decode_step(case)
    for b in range(spec.B):
        ids, o = bf_decode_seq(case, b)
        assert res["ids"][b].tolist() == ids
        assert within(res["out"][b][0], o, "bf16"), b
    assert any((int(t) + 1) % spec.m == 0 for t in case["pos"])   # an entry is pooled
    for mistake in ("raw_window", "no_qrope", "out_sign"):
        assert any(not within(res["out"][b][0], bf_decode_seq(case, b, mistake)[1], "bf16")
                   for b in range(spec.B)), mistake


def _rotate_rows(rows, positions, rd):
    return np.stack([bf_rope(r, float(p), rd) for r, p in zip(rows, positions)])


def shifted_decode_cases(shift_blocks: int):
    """A one-sequence decode step with RMSNorm + RoPE everywhere, and the same step with every
    position moved by shift_blocks * m: the cached entries and window rows carry the rotation
    of their own positions (the entries' indices move by shift_blocks; the new slots in front
    have zero indexer keys and are never selected), the queries, gates, raw new rows and tails
    are the same. Storage fp32."""
    spec = datagen.CaseSpec(917, "decode", dtype="f32", B=1, L=256, m=4, H_I=8, d_I=16, H=4,
                            D=32, K=8, W=8, w_cap=16)
    a = datagen.make_case(spec)
    a["w"] = a["w"].abs()                  # scores >= 0: zero-key slots rank last
    rd = 16
    a.update(kv_rope_dim=rd, q_rope_dim=rd, out_rope_dim=rd,
             kv_gamma=datagen.tensor(917, 40, (32,), "f32", 0.3).abs() + 0.5,
             q_gamma=[datagen.tensor(917, 41, (32,), "f32", 0.3).abs() + 0.5])
    m, E, wc = spec.m, spec.entries, spec.w_cap
    t_a = int(a["pos"][0])
    kv_u, ki_u = f64(a["kv"][0]), f64(a["k_idx"][0])
    ring_u = f64(a["rings"][0][0])
    ring_pos = {p: ring_u[p % wc] for p in range(t_a - wc + 1, t_a)}   # rows before t

    def build(delta_blocks):
        d = delta_blocks * m
        c = dict(a)
        sp = dataclasses.replace(spec, L=spec.L + d)
        kv = np.zeros((1, E + delta_blocks, 32))
        ki = np.zeros((1, E + delta_blocks, 16))
        kv[0, delta_blocks:] = _rotate_rows(kv_u, [m * (e + 1) - 1 + d for e in range(E)], rd)
        ki[0, delta_blocks:] = ki_u
        ring = np.zeros((1, wc, 32))
        for p, r in ring_pos.items():
            ring[0, (p + d) % wc] = bf_rope(r, float(p + d), rd)
        c.update(spec=sp, pos=torch.tensor([t_a + d]), kv=torch.from_numpy(kv).float(),
                 k_idx=torch.from_numpy(ki).float(), rings=[torch.from_numpy(ring).float()])
        return c

    return build(0), build(shift_blocks)


def test_decode_step_outputs_depend_only_on_distances():
    # [CoD "Key and value are the same vector"]: with every key/value row rotated at its own
    # position, the query at +t and the output back at -t, shifting every position by the same
    # amount leaves the step's output unchanged
    a, b = shifted_decode_cases(shift_blocks=37)
    ra, rb = pipeline.decode_step(a), pipeline.decode_step(b)
    assert rb["ids"][0].tolist() == [i + 37 for i in ra["ids"][0].tolist()]
    oa, ob = ra["out"][0][0], rb["out"][0][0]
    np.testing.assert_allclose(ob, oa, rtol=0, atol=2e-6 * np.abs(oa).max())
    # the rotations are live: without the output's inverse RoPE the two differ
    a2, b2 = dict(a, out_rope_dim=0), dict(b, out_rope_dim=0)
    o2a, o2b = pipeline.decode_step(a2)["out"][0][0], pipeline.decode_step(b2)["out"][0][0]
    assert np.abs(o2a - o2b).max() > 1e-2 * np.abs(o2a).max()


# ---- the overlapped compressor inside the decode step ----------------------------------
def c4a_stream_case(m: int, t: int, seq: dict):
    """A one-sequence fp32 decode step at position t whose compressor state is what a stream of
    steps over the rows in ``seq`` (xa, za, xb, zb: [T, D] for positions 0 .. T-1) leaves: the
    a tail holds the current block's rows before t (its new slot zero), the b ring the b rows of
    positions p < t at row p % 2m back to the previous block's start; ring rows never written
    hold random stale values."""
    spec = datagen.CaseSpec(921, "decode", dtype="f32", B=1, L=seq["xa"].shape[0], m=m, H_I=4,
                            d_I=16, H=2, D=seq["xa"].shape[1], K=4, W=4, w_cap=8,
                            compressor="c4a")
    case = datagen.make_case(spec)
    s0 = t - t % m
    x_tail = np.zeros((1, m, spec.D), np.float32)
    z_tail = np.zeros((1, m, spec.D), np.float32)
    for p in range(s0, t):
        x_tail[0, p - s0], z_tail[0, p - s0] = seq["xa"][p], seq["za"][p]
    xb_tail = case["xb_tail"].numpy().copy()     # stale rows as drawn
    zb_tail = case["zb_tail"].numpy().copy()
    for p in range(max(s0 - m, 0), t):
        xb_tail[0, p % (2 * m)], zb_tail[0, p % (2 * m)] = seq["xb"][p], seq["zb"][p]
    case.update(pos=torch.tensor([t]), x_tail=torch.from_numpy(x_tail),
                z_tail=torch.from_numpy(z_tail), xb_tail=torch.from_numpy(xb_tail),
                zb_tail=torch.from_numpy(zb_tail),
                x_new=torch.from_numpy(seq["xa"][t][None].copy()),
                z_new=torch.from_numpy(seq["za"][t][None].copy()),
                xb_new=torch.from_numpy(seq["xb"][t][None].copy()),
                zb_new=torch.from_numpy(seq["zb"][t][None].copy()),
                bias=torch.from_numpy(seq["ba"].copy()), bias_b=torch.from_numpy(seq["bb"].copy()))
    return case


@pytest.mark.parametrize("m", [1, 2, 4])
def test_decode_step_c4a_entries_match_the_chunk_compressor(m):
    # [CoD "The compressor has two streams and they overlap"]: entry e of a sequence pools the a
    # rows of block e and the b rows of block e - 1; stepping token by token through the decode
    # state must give the entries the chunk compressor gives over the whole sequence at once
    T, D = 6 * m, 16
    g = np.random.default_rng(5150 + m)
    seq = {k: g.standard_normal((T, D)).astype(np.float32) for k in ("xa", "za", "xb", "zb")}
    seq["ba"] = (0.5 * g.standard_normal((m, D))).astype(np.float32)
    seq["bb"] = (0.5 * g.standard_normal((m, D))).astype(np.float32)
    want = csa.compress_c4a(seq["xa"], seq["za"], seq["xb"], seq["zb"], seq["ba"], seq["bb"], m)
    # plausible mistakes: the b rows of the entry's own block, no b-part, the single stream
    own = np.stack([csa.compress_c4a(seq["xa"][m * e:m * e + m], seq["za"][m * e:m * e + m],
                                     seq["xb"][:m], seq["zb"][:m], seq["ba"], seq["bb"], m,
                                     Xb_prev=seq["xb"][m * e:m * e + m],
                                     Zb_prev=seq["zb"][m * e:m * e + m])[0] for e in range(6)])
    single = csa.compress(seq["xa"], seq["za"], seq["ba"], m)
    for e in range(6):
        t = m * e + m - 1
        got = pipeline.decode_step(c4a_stream_case(m, t, seq))["kv_new_exact"][0]
        np.testing.assert_allclose(got, want[e], rtol=0, atol=1e-12)
        if e > 0:
            assert np.abs(got - own[e]).max() > 1e-3
            assert np.abs(got - single[e]).max() > 1e-3
        else:   # the sequence's first entry has no previous block: a rows only
            np.testing.assert_allclose(got, single[0], rtol=0, atol=1e-12)
    if m > 1:   # a step that does not complete a block pools nothing
        assert pipeline.decode_step(c4a_stream_case(m, 2 * m - 2, seq))["kv_new"] == {}


def test_decode_step_c4a_state_drawn_by_datagen():
    # the b ring datagen draws for a decode step holds the previous block's rows where the step
    # reads them: its entry equals the chunk compressor over the drawn rows of both blocks
    spec = datagen.CaseSpec(922, "decode", dtype="f32", B=3, L=4 * 300, m=4, H_I=4, d_I=16, H=2,
                            D=16, K=4, W=4, w_cap=8, ragged=True, compressor="c4a")
    case = datagen.make_case(spec)
    res = pipeline.decode_step(case)
    m = spec.m
    n_pooled = 0
    for b in range(spec.B):
        t = int(case["pos"][b])
        if (t + 1) % m:
            continue
        n_pooled += 1
        e = (t + 1) // m - 1
        xa = f64(case["x_tail"][b]).copy()
        za = f64(case["z_tail"][b]).copy()
        xa[m - 1], za[m - 1] = f64(case["x_new"][b]), f64(case["z_new"][b])
        h = ((e - 1) % 2) * m
        xb, zb = f64(case["xb_tail"][b])[h:h + m], f64(case["zb_tail"][b])[h:h + m]
        # entry 1 of a two-block chunk pools block 1's a rows with block 0's b rows
        want = csa.compress_c4a(np.concatenate([xa, xa]), np.concatenate([za, za]),
                                np.concatenate([xb, xb]), np.concatenate([zb, zb]),
                                f64(case["bias"]), f64(case["bias_b"]), m)[1]
        np.testing.assert_allclose(res["kv_new_exact"][b], want, rtol=0, atol=1e-12)
    assert n_pooled >= 1
