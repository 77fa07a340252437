"""Score-gap enforcement for generated inputs -- TEST INFRASTRUCTURE ONLY.

Bit-exact Top-K parity needs a unique selection that fp32 rounding cannot flip. For
every checked query whose visible count exceeds K, the K-th and (K+1)-th highest float64
scores a > b must satisfy  a - b > 1e-3 * max(|a|, |b|, mean|S|);  otherwise the query's
gate (or, in the tiny workload, its indexer query and gate together) is redrawn from the
seeded generator with the next attempt number. Scores come from the oracle only.
"""
from __future__ import annotations

import numpy as np

import datagen

from . import csa
from .pipeline import cached_index_key, f64, i64, index_query

REL_GAP = 1e-3
MAX_ATTEMPTS = 2000
MAX_BLOCK_ATTEMPTS = 50000


def gap_ok(scores: np.ndarray, K: int) -> bool:
    """True when the K-th and (K+1)-th largest scores are separated by the required gap
    (always true when there are at most K scores)."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    if n <= K:
        return True
    part = -np.partition(-s, (K - 1, K))
    a, b = part[K - 1], part[K]
    return (a - b) > REL_GAP * max(abs(a), abs(b), float(np.abs(s).mean()))


REL_MID = 1e-4


def gap_ok_bf16(scores: np.ndarray, K: int) -> bool:
    """For a selection over BF16-rounded scores: ties at the K-th bf16 value are broken by id,
    so the selection is unique; it is robust to fp32 rounding when no score that rounds to
    the K-th bf16 value or a neighbour of it lies within REL_MID * max(|s|, mean|S|) of a bf16
    rounding midpoint (always true when there are at most K scores)."""
    s = csa.round_f32(np.asarray(scores, dtype=np.float64))
    n = s.shape[0]
    if n <= K:
        return True
    b = csa.round_bf16(s)
    vk = -np.partition(-b, K - 1)[K - 1]
    _, e = np.frexp(max(abs(vk), 2.0 ** -126))
    ulp = np.ldexp(1.0, e - 8)
    near = np.abs(s - vk) <= 2.5 * ulp
    if not near.any():
        return True
    sn, bn = s[near], b[near]
    _, eb = np.frexp(np.maximum(np.abs(bn), 2.0 ** -126))
    q = np.ldexp(1.0, eb - 8)                 # spacing at |b|; below a power of two it halves
    lo_q = np.where(np.abs(bn) == np.ldexp(0.5, eb), q / 2, q)
    up = np.where(bn >= 0, q, lo_q)
    down = np.where(bn >= 0, lo_q, q)
    dist = np.minimum(np.abs(sn - (bn + up / 2)), np.abs(sn - (bn - down / 2)))
    scale = np.maximum(np.abs(sn), float(np.abs(s).mean()))
    return bool(np.all(dist > REL_MID * scale))


def _blocks_gap(S: np.ndarray, spec) -> np.ndarray:
    """gap_ok on the block maxima at rank max_blocks, per column of S [n, k]. The maxima are
    taken over the whole batch at once here (a search aid); the gate that is kept is checked
    again with csa.block_maxima itself."""
    S = csa.round_f32(S)
    n, k = S.shape
    bs = spec.block_size
    nb = (n + bs - 1) // bs
    P = np.full((nb * bs, k), -np.inf)
    P[:n] = S
    bm = P.reshape(nb, bs, k).max(axis=1)
    return np.array([gap_ok(bm[:, j], spec.max_blocks) for j in range(k)])


def _fix_w(spec, R: np.ndarray, K: int, which: str, b: int, current, ok=gap_ok) -> tuple[object, int]:
    """Redraw a gate row until the scores R @ w have the gap at rank K (``ok`` the rule)."""
    w = current
    attempt = 0
    while not ok(R @ f64(w), K):
        attempt += 1
        if attempt > MAX_ATTEMPTS:
            raise RuntimeError(f"no gap after {MAX_ATTEMPTS} redraws ({which}, row {b})")
        w = datagen.redraw_w(spec, which, b, attempt)
    return w, attempt


def enforce_decode(case: dict, seqs=None) -> dict:
    """Decode step inputs: fix w (flat) or w then w2 (hierarchical) per sequence."""
    spec = case["spec"]
    m, E = spec.m, spec.entries
    pos = i64(case["pos"])
    seqs = range(spec.B) if seqs is None else seqs
    redraws = {}
    bias_i = f64(case["bias_i"])
    for b in seqs:
        t = int(pos[b])
        n = csa.n_visible(t, m, E)
        keys = f64(case["k_idx"][b][:n]).copy()
        if (t + 1) % m == 0:
            xi = f64(case["xi_tail"][b]).copy()
            zi = f64(case["zi_tail"][b]).copy()
            xi[t % m] = f64(case["xi_new"][b])
            zi[t % m] = f64(case["zi_new"][b])
            e = (t + 1) // m - 1
            if e < n:
                keys[e] = cached_index_key(
                    case, csa.store(csa.compress(xi, zi, bias_i, m)[0], spec.dtype))
        R = csa.head_relu(index_query(case, case["q_idx"][b]), keys)
        if spec.block_size > 0:
            # stage 1: the block maxima must separate at rank max_blocks. With tens of
            # thousands of blocks that gap is rare (about one gate in a thousand), so the
            # redraws are scored in batches; the first passing attempt is kept, as a
            # one-by-one search would.
            w = case["w"][b]
            attempt = 0
            while not gap_ok(csa.block_maxima(R @ f64(w), spec.block_size), spec.max_blocks):
                ok = np.zeros(0, bool)
                base = attempt + 1
                while base <= MAX_BLOCK_ATTEMPTS:
                    ws = [datagen.redraw_w(spec, "w", b, a)
                          for a in range(base, min(base + 64, MAX_BLOCK_ATTEMPTS + 1))]
                    ok = _blocks_gap(R @ np.stack([f64(x) for x in ws], axis=1), spec)
                    if ok.any():
                        break
                    base += len(ws)
                if not ok.any():
                    raise RuntimeError(f"no block gap after {MAX_BLOCK_ATTEMPTS} redraws (row {b})")
                attempt = base + int(np.argmax(ok))
                w = ws[int(np.argmax(ok))]
            case["w"][b] = w
            s1 = R @ f64(w)
            pool = csa.candidate_pool(s1, spec.block_size, spec.max_blocks)
            R2 = csa.head_relu(f64(case["q_idx2"][b]), keys[pool])
            w2, a2 = _fix_w(spec, R2, spec.K, "w2", b, case["w2"][b])
            case["w2"][b] = w2
            redraws[b] = (attempt, a2)
        else:
            rule = gap_ok_bf16 if case.get("score_format") == "bf16" else gap_ok
            w, a = _fix_w(spec, R, spec.K, "w", b, case["w"][b], rule)
            case["w"][b] = w
            redraws[b] = a
    return redraws


def enforce_rows(case: dict, rows, keys_for_row) -> dict:
    """Per query row (b, i): fix w[b, i] so the visible scores separate at rank K.
    ``keys_for_row(b, i)`` returns the float64 visible keys of that row."""
    spec = case["spec"]
    redraws = {}
    for b, i in rows:
        keys = keys_for_row(b, i)
        R = csa.head_relu(f64(case["q_idx"][b, i]), keys)
        row_id = b * 1_000_003 + i
        w = case["w"][b, i]
        attempt = 0
        while not gap_ok(R @ f64(w), spec.K):
            attempt += 1
            if attempt > MAX_ATTEMPTS:
                raise RuntimeError("no gap")
            w = datagen.redraw_w(spec, "w", row_id, attempt)
        case["w"][b, i] = w
        redraws[(b, i)] = attempt
    return redraws


def enforce_prefill(case: dict, rows, ki_c=None) -> dict:
    """Chunked prefill: fix the gates of the checked query rows (keys include the chunk's
    own pooled entries: by default the oracle's, or the stored chunk keys ki_c [B, chunk/m,
    d_I] a caller passes, e.g. the ones another implementation pooled)."""
    spec = case["spec"]
    if ki_c is None:
        ki_c = csa.store(csa.compress(f64(case["xi_chunk"]), f64(case["zi_chunk"]),
                                      f64(case["bias_i"]), spec.m), spec.dtype)
    ki_c = f64(ki_c)
    e0 = (spec.L - spec.chunk) // spec.m
    qp = i64(case["q_pos"])
    cache = {}

    def keys_for_row(b, i):
        if b not in cache:
            k = f64(case["k_idx"][b]).copy()
            k[e0:e0 + ki_c.shape[1]] = ki_c[b]
            cache.clear()
            cache[b] = k
        n = csa.n_visible(int(qp[b, i]), spec.m, spec.entries)
        return cache[b][:n]

    return enforce_rows(case, rows, keys_for_row)


def enforce_tiny(case: dict, rows=None) -> dict:
    """Tiny workload: redraw (q_idx row, w row) jointly until the gap holds (with 4 heads an
    all-zero tie among entries cannot be split by the gate alone)."""
    spec = case["spec"]
    qp = i64(case["q_pos"])
    B, Q = qp.shape
    rows = rows if rows is not None else [(b, i) for b in range(B) for i in range(Q)]
    redraws = {}
    E = spec.L // spec.m
    for b, i in rows:
        n = csa.n_visible(int(qp[b, i]), spec.m, E)
        if n <= spec.K:
            continue
        keys = f64(case["k_idx"][b][:n])
        attempt = 0
        q, w = case["q_idx"][b, i], case["w"][b, i]
        while not gap_ok(csa.index_scores(f64(q), f64(w), keys), spec.K):
            attempt += 1
            if attempt > MAX_ATTEMPTS:
                raise RuntimeError("no gap")
            q, w = datagen.redraw_qw(spec, b * 1_000_003 + i, attempt)
        case["q_idx"][b, i] = q
        case["w"][b, i] = w
        redraws[(b, i)] = attempt
    return redraws
