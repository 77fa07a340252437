"""GPU parity of each libcsa call against the float64 oracle, at sizes the oracle finishes in
seconds that still span several tiles and a ragged tail. All calls go through the C ABI."""
import math

import numpy as np
import pytest
import torch

import datagen
import sparse_long_context_csa_amd as csa
from gpu_helpers import (assert_ids, assert_pooled, assert_rows_close, assert_scores, bf16_ulp, dev,
                         fix_gaps, pooled_xmax)
from oracle import csa as ocsa
from oracle import gaps, pipeline
from oracle.pipeline import f64, i64

pytestmark = pytest.mark.gpu
CID = 7000


def T(tid, shape, dtype="bf16", scale=1.0, *extra):
    return datagen.tensor(CID, tid, shape, dtype, scale, 0, *extra)


# ------------------------------------------------------------------------------ compress
@pytest.mark.parametrize("dtype,m,dim,n_tok,n_seq", [
    ("bf16", 4, 512, 4096, 2), ("bf16", 1, 128, 37, 3), ("bf16", 2, 64, 130, 1),
    ("bf16", 8, 136, 64, 2), ("f32", 4, 64, 2048, 1), ("f32", 16, 8, 32, 2),
    # long entries (HCA's m' = 128): the workgroup-per-entry pooling with merged partials
    ("bf16", 128, 512, 1024, 2), ("bf16", 17, 8, 34, 2), ("bf16", 100, 136, 300, 1),
    ("f32", 32, 64, 128, 2), ("f32", 128, 40, 256, 1),
])
def test_compress(dtype, m, dim, n_tok, n_seq):
    x = T(1, (n_seq, n_tok, dim), dtype, 1.0, m, dim)
    z = T(2, (n_seq, n_tok, dim), dtype, 1.0, m, dim)
    b = T(3, (m, dim), dtype, 0.5, m, dim)
    out = csa.compress(dev(x), dev(z), dev(b), m)
    torch.cuda.synchronize()
    ref64 = ocsa.compress(f64(x), f64(z), f64(b), m)
    got = f64(out.cpu())
    if dtype == "bf16":
        # fp32 arithmetic then one RNE store
        assert_pooled(got, ref64, pooled_xmax(f64(x), m), "compress", m=m)
        frac = np.mean(got == ocsa.round_bf16(ref64))
        assert frac > 0.999, frac
    else:
        tol = max(2e-6, 2.0 * (m + 8) * 2.0 ** -24)
        np.testing.assert_allclose(got, ref64, rtol=tol, atol=tol * np.abs(f64(x)).max())


def test_compress_into_cache_offset():
    m, dim, n_tok, e_cap, e0 = 4, 512, 256, 200, 100
    x, z, b = T(4, (2, n_tok, dim)), T(5, (2, n_tok, dim)), T(6, (m, dim))
    cache = torch.zeros(2, e_cap, dim, dtype=torch.bfloat16, device="cuda")
    csa.compress(dev(x), dev(z), dev(b), m, out=cache[:, e0:], out_seq_stride=e_cap * dim)
    torch.cuda.synchronize()
    got = f64(cache.cpu())
    exact = ocsa.compress(f64(x), f64(z), f64(b), m)
    assert np.all(got[:, :e0] == 0) and np.all(got[:, e0 + n_tok // m:] == 0)
    assert_pooled(got[:, e0:e0 + n_tok // m], exact, pooled_xmax(f64(x), m), "cache offset")


# ---------------------------------------------------------- overlapped two-stream compressor
@pytest.mark.parametrize("dtype,m,dim,n_tok,n_seq,prev", [
    ("bf16", 4, 512, 4096, 2, False),      # the prefill chunk's shape, start of the sequence
    ("bf16", 4, 512, 1024, 3, True),       # a chunk in the middle of the sequence
    ("bf16", 1, 128, 96, 2, True),
    ("bf16", 2, 256, 128, 2, True),
    ("bf16", 2, 256, 128, 1, False),
    ("bf16", 8, 64, 512, 1, False),
    ("bf16", 16, 136, 256, 2, True),       # m = 16, dim not a multiple of 64
    ("f32", 4, 64, 256, 2, True),
    ("f32", 3, 8, 48, 1, False),
])
def test_compress_c4a(dtype, m, dim, n_tok, n_seq, prev):
    sh = (n_seq, n_tok, dim)
    xa, za = T(40, sh, dtype, 1.0, m, dim), T(41, sh, dtype, 2.0, m, dim)
    xb, zb = T(42, sh, dtype, 1.0, m, dim), T(43, sh, dtype, 2.0, m, dim)
    ba, bb = T(44, (m, dim), dtype, 0.5, m, dim), T(45, (m, dim), dtype, 0.5, m, dim)
    xp = T(46, (n_seq, m, dim), dtype, 1.0, m, dim) if prev else None
    zp = T(47, (n_seq, m, dim), dtype, 2.0, m, dim) if prev else None
    out = csa.compress_c4a(dev(xa), dev(za), dev(xb), dev(zb), dev(ba), dev(bb), m,
                           xb_prev=dev(xp), zb_prev=dev(zp))
    torch.cuda.synchronize()
    ref64 = ocsa.compress_c4a(f64(xa), f64(za), f64(xb), f64(zb), f64(ba), f64(bb), m,
                              None if xp is None else f64(xp), None if zp is None else f64(zp))
    got = f64(out.cpu())
    # each entry's 2m rows: a-part of its block, b-part of the block before
    xab = np.abs(f64(xa)).reshape(n_seq, n_tok // m, m, dim).max(axis=2)
    xbb = np.abs(f64(xb)).reshape(n_seq, n_tok // m, m, dim).max(axis=2)
    xmax = xab.copy()
    xmax[:, 1:] = np.maximum(xmax[:, 1:], xbb[:, :-1])
    if xp is not None:
        xmax[:, 0] = np.maximum(xmax[:, 0], np.abs(f64(xp)).max(axis=1))
    if dtype == "bf16":
        assert_pooled(got, ref64, xmax, "compress_c4a")
        frac = np.mean(got == ocsa.round_bf16(ref64))
        assert frac > 0.999, frac
    else:
        # fp32 online softmax over 2m rows: a few ulp of the largest row per entry
        ratio = float((np.abs(got - ref64) / xmax).max())
        assert ratio < 4e-6, ratio


def test_compress_c4a_chunks_into_a_cache():
    """Two chunks of one sequence written into a cache at entry offsets, the second with the
    first chunk's last b-stream block as its previous block: the cache equals the whole."""
    m, dim, n_tok, e_cap = 4, 512, 512, 300
    sh = (1, 2 * n_tok, dim)
    xa, za, xb, zb = (T(50 + i, sh) for i in range(4))
    ba, bb = T(54, (m, dim), "bf16", 0.5), T(55, (m, dim), "bf16", 0.5)
    cache = torch.zeros(1, e_cap, dim, dtype=torch.bfloat16, device="cuda")
    g = [dev(t) for t in (xa, za, xb, zb)]
    n_ent = n_tok // m
    csa.compress_c4a(*(t[:, :n_tok] for t in g), dev(ba), dev(bb), m, out=cache,
                     out_seq_stride=e_cap * dim)
    csa.compress_c4a(*(t[:, n_tok:] for t in g), dev(ba), dev(bb), m,
                     xb_prev=g[2][:, n_tok - m:n_tok].contiguous(),
                     zb_prev=g[3][:, n_tok - m:n_tok].contiguous(),
                     out=cache[:, n_ent:], out_seq_stride=e_cap * dim)
    torch.cuda.synchronize()
    got = f64(cache.cpu())
    exact = ocsa.compress_c4a(f64(xa), f64(za), f64(xb), f64(zb), f64(ba), f64(bb), m)
    assert np.all(got[:, 2 * n_ent:] == 0)
    xm = np.abs(np.concatenate([f64(xa), f64(xb)], axis=-1)).max()
    assert_pooled(got[:, :2 * n_ent], exact, xm, "c4a chunks")


# ------------------------------------------------------------- per-head RMSNorm + partial RoPE
@pytest.mark.parametrize("dtype,rows,heads,dim,rope_dim,flags", [
    ("bf16", 4, 64, 512, 64, "norm+rope"),     # decode queries at 1M positions
    ("bf16", 300, 1, 512, 64, "norm+rope"),    # compressed entries (one head)
    ("bf16", 4, 64, 512, 64, "inverse"),       # the attention output
    ("bf16", 7, 3, 136, 32, "rope"),
    ("bf16", 5, 2, 64, 64, "norm"),
    ("f32", 9, 4, 128, 64, "norm+rope"),
    ("f32", 3, 2, 8, 2, "inverse"),
])
def test_norm_rope(dtype, rows, heads, dim, rope_dim, flags):
    x = T(60, (rows, heads, dim), dtype, 1.0, dim)
    gamma = T(61, (dim,), dtype, 0.5, dim) if "norm" in flags else None
    g = np.random.default_rng(dim + rows)
    pos = torch.from_numpy(g.integers(0, 1 << 20, size=rows).astype(np.int64))
    use_pos = "rope" in flags or flags == "inverse"
    out = csa.norm_rope(dev(x), dev(gamma), dev(pos) if use_pos else None, rope_dim=rope_dim,
                        inverse=flags == "inverse")
    torch.cuda.synchronize()
    ref = f64(x)
    if gamma is not None:
        ref = ocsa.rms_norm(ref, f64(gamma), 1e-6)
    if use_pos:
        p = f64(pos)[:, None] * (-1.0 if flags == "inverse" else 1.0)
        ref = ocsa.rope(ref, p, rope_dim)
    got = f64(out.cpu())
    # fp32 arithmetic then one rounding to T: half a storage spacing plus the fp32 error of
    # the mean square (at most dim * 2^-24 relative, halved by the square root) on the largest
    # magnitude in the vector
    vmax = np.abs(ref).max(axis=-1, keepdims=True)
    spacing = bf16_ulp(np.maximum(np.abs(got), np.abs(ref))) if dtype == "bf16" else 0.0
    tol = 0.5 * spacing + (dim * 2.0 ** -24 + 1e-6) * vmax
    assert np.all(np.abs(got - ref) <= tol), float(np.max(np.abs(got - ref) - tol))


def test_norm_rope_in_place_round_trip():
    # rotate in place, then rotate back at -pos: the rotated part returns to the input within
    # two roundings; the rest is untouched bit for bit
    x = T(62, (8, 64, 512), "f32", 1.0)
    pos = torch.from_numpy(np.arange(8, dtype=np.int64) * 131071)
    y = dev(x).clone()
    csa.norm_rope(y, pos=dev(pos), out=y)
    csa.norm_rope(y, pos=dev(pos), inverse=True, out=y)
    torch.cuda.synchronize()
    got = y.cpu()
    assert torch.equal(got[..., :448], x[..., :448])
    assert torch.allclose(got[..., 448:], x[..., 448:], rtol=0, atol=2e-6)


# ------------------------------------------------------------------------------ index + top-k
def index_case(B, Q, E, H, d, dtype, t_lo, t_hi, m=4, seed=0):
    q = T(10, (B, Q, H, d), dtype, 1 / math.sqrt(d), seed)
    w = T(11, (B, Q, H), dtype, 1 / math.sqrt(H), seed).float()
    k = T(12, (B, E, d), dtype, 1 / math.sqrt(d), seed)
    g = np.random.default_rng(seed)
    pos = torch.from_numpy(g.integers(t_lo, t_hi, size=(B, Q)).astype(np.int64))
    return q, w, k, pos


def check_index(q, w, k, pos, m, K, e_count=None, cand=None, dtype="bf16", rows=None):
    fix_gaps(CID, q, w, k, pos, e_count, m, K, cand=cand, dtype=dtype)
    res = csa.index_topk(dev(q), dev(w), dev(k), dev(pos), m, K, e_count=dev(e_count),
                         cand=dev(cand), want_scores=True, want_all=True)
    idx, osc, alls = [x.cpu() for x in res]
    B, Q = pos.shape
    ref = pipeline.index_topk(q, w, k, pos, e_count, m, K, rows=rows, cand=cand)
    for (b, i), (ids, s, sid) in ref.items():
        assert_ids(idx[b, i].numpy(), ids, f"row {(b, i)}")
        A = ocsa.score_scale(f64(q[b, i]), f64(w[b, i]), f64(k[b])[sid]) if sid.size else np.zeros(0)
        if cand is None:
            assert_scores(alls[b, i, :sid.size].numpy(), s, A, what=f"scores {(b, i)}")
            assert np.all(np.isneginf(alls[b, i, sid.size:].numpy()))
        else:
            c = i64(cand[b, i])
            pos_of = {int(v): j for j, v in enumerate(c) if 0 <= v}
            got = np.array([alls[b, i, pos_of[int(v)]].item() for v in sid])
            assert_scores(got, s, A, what=f"cand scores {(b, i)}")
        sel = ids >= 0
        exp = dict(zip(sid.tolist(), s.tolist()))
        got_s = osc[b, i].numpy()
        for j in np.nonzero(sel)[0]:
            e = exp[int(ids[j])]
            assert abs(got_s[j] - e) <= 1e-3 * A[list(sid).index(ids[j])] + 1e-30
        assert np.all(np.isneginf(got_s[~sel]))


def test_index_decode_fast_path():
    # 64x128 bf16, few query rows: MFMA scan; ragged visible counts incl. partial tiles
    q, w, k, pos = index_case(3, 1, 5000, 64, 128, "bf16", 4 * 700, 4 * 5000)
    pos[0, 0] = 4 * 5000 - 1      # every entry visible
    pos[1, 0] = 2049              # 512 visible, K = 512 -> exactly all
    check_index(q, w, k, pos, 4, 512)


def test_index_rows_of_many_groups():
    # rows of 16K-32K visible entries (no segments): the select's bound takes one 16-position
    # maximum per group, more than two groups per thread (loaded in one round), or, below 16K
    # positions, the score groups of the general loop
    q, w, k, pos = index_case(3, 1, 30000, 64, 128, "bf16", 4 * 14000, 4 * 30000, seed=31)
    pos[0, 0] = 4 * 30000 - 1     # 30,000 visible: 1,875 groups
    pos[1, 0] = 4 * 20000 + 2     # 20,000 visible: 1,250 groups
    pos[2, 0] = 4 * 15000 + 1     # 15,000 visible: under 2K groups of 16, the score path
    check_index(q, w, k, pos, 4, 512)


def test_index_decode_small_visible():
    q, w, k, pos = index_case(2, 2, 300, 64, 128, "bf16", -3, 60, seed=1)
    pos[0, 0] = -1                # nothing visible
    pos[0, 1] = 2                 # t < m: nothing visible
    pos[1, 0] = 3                 # one entry
    check_index(q, w, k, pos, 4, 16)


def test_index_e_count_caps_visibility():
    q, w, k, pos = index_case(2, 1, 3000, 64, 128, "bf16", 11990, 12000, seed=2)
    e_count = torch.tensor([1000, 2999], dtype=torch.int32)
    check_index(q, w, k, pos, 4, 128, e_count=e_count)


def test_index_long_rows_segmented_select():
    # more candidates than one workgroup holds (32,768): segment + merge levels
    q, w, k, pos = index_case(2, 1, 70000, 64, 128, "bf16", 4 * 70000 - 1, 4 * 70000, seed=3)
    check_index(q, w, k, pos, 4, 512)


def test_index_segments_ragged_rows():
    # long decode rows leave candidate segments from the scan; a short row of the same batch
    # (<= 32,768 visible) takes the single-row select inside the same launch
    E = 100000
    q, w, k, pos = index_case(3, 1, E, 64, 128, "bf16", 0, 1, seed=12)
    pos[0, 0] = 4 * 20000 - 1
    pos[1, 0] = 4 * 50000 + 2
    pos[2, 0] = 4 * E - 1
    check_index(q, w, k, pos, 4, 512)


def test_index_segments_clustered_winners():
    # keys of one stretch doubled (ReLU is positively homogeneous: exactly doubled scores), so
    # most of the Top-512 sit in a few chunks whose own thresholds lie above the K-th key:
    # the select must notice and fall back to streaming the row above its bound
    E = 90000
    q, w, k, pos = index_case(2, 1, E, 64, 128, "bf16", 4 * E - 1, 4 * E, seed=13)
    k[0, 30000:31500] = (k[0, 30000:31500].float() * 2).to(k.dtype)
    k[1, 100:400] = (k[1, 100:400].float() * 2).to(k.dtype)
    check_index(q, w, k, pos, 4, 512)


@pytest.mark.parametrize("B,E,K", [(3, 1200, 64), (1, 40000, 512)], ids=["scores", "segments"])
def test_index_odd_work_items(B, E, K):
    # an odd count of (row, chunk) work items (15 and 157 chunks of 256 positions), fewer than
    # the persistent grid's blocks: the scan's item loop and the segments of a row whose item
    # count is odd
    q, w, k, pos = index_case(B, 1, E, 64, 128, "bf16", 4 * E - 1, 4 * E, seed=21)
    check_index(q, w, k, pos, 4, K)


def test_index_blocks_own_topk_segments():
    # stage 1 of the hierarchical indexer with the row's own Top-K over long rows
    B, E, bs, mb, K = 2, 50000, 8, 64, 512
    q, w, k, pos = index_case(B, 1, E, 64, 128, "bf16", E - 5, E, m=1, seed=14)
    fix_gaps(CID, q, w, k, pos, None, 1, K)
    pool, idx = csa.index_blocks(dev(q), dev(w), dev(k), dev(pos), 1, bs, mb, top_k=K)
    idx = idx.cpu()
    ref = pipeline.index_topk(q, w, k, pos, None, 1, K)
    for (b, i), (ids, _, _) in ref.items():
        assert_ids(idx[b, i].numpy(), ids, f"row {(b, i)}")


@pytest.mark.parametrize("n_dup,contiguous", [(600, False), (600, True), (9000, False)])
def test_index_exact_ties(n_dup, contiguous):
    """Exact score ties across the K-th place: n_dup copies of the best key row (scaled by 2,
    exact in bf16) score identically on both sides, so the K places go to the lowest ids.
    Spread copies exercise the LDS list; a contiguous run overflows one filter segment and a
    9,000-copy spread overflows the list: both take the streaming select."""
    E, K = 40000, 512
    q, w, k, pos = index_case(1, 1, E, 64, 128, "bf16", 4 * E - 1, 4 * E, seed=11)
    s = ocsa.index_scores(f64(q[0, 0]), f64(w[0, 0]), f64(k[0]))
    best = int(np.argmax(s))
    g = np.random.default_rng(11)
    if contiguous:
        at = np.arange(7000, 7000 + n_dup)
    else:
        at = np.sort(g.choice(E, size=n_dup, replace=False))
    k[0, at] = (k[0, best].float() * 2).to(k.dtype)
    res = csa.index_topk(dev(q), dev(w), dev(k), dev(pos), 4, K, want_scores=True)
    idx, osc = [x.cpu() for x in res]
    ref = pipeline.index_topk(q, w, k, pos, None, 4, K)
    ids = ref[(0, 0)][0]
    assert np.array_equal(ids, np.sort(at)[:K])
    assert_ids(idx[0, 0].numpy(), ids, "ties")
    assert np.all(osc[0, 0].numpy() == osc[0, 0, 0].item())


def test_index_prefill_fast_path():
    # >= 16 query rows: LDS-tiled MFMA scan; consecutive positions, causal edge inside tiles
    B, Q, E = 1, 40, 3000
    q, w, k, _ = index_case(B, Q, E, 64, 128, "bf16", 0, 1, seed=4)
    pos = torch.arange(4 * E - Q - 5, 4 * E - 5, dtype=torch.int64).view(1, Q)
    check_index(q, w, k, pos, 4, 512)


def test_index_candidates():
    q, w, k, pos = index_case(2, 1, 4000, 64, 128, "bf16", 15000, 16000, seed=5)
    g = np.random.default_rng(5)
    cand = np.full((2, 1, 1500), -1, np.int32)
    for b in range(2):
        c = np.sort(g.choice(4000, size=1400, replace=False))
        cand[b, 0, :1400] = c      # some beyond the visible count: ignored
    cand = torch.from_numpy(cand)
    check_index(q, w, k, pos, 4, 256, cand=cand)


@pytest.mark.parametrize("H,d,dtype", [(4, 32, "f32"), (16, 64, "bf16"), (64, 128, "f32")])
def test_index_generic_path(H, d, dtype):
    q, w, k, pos = index_case(2, 3, 700, H, d, dtype, 4 * 100, 4 * 700, seed=6)
    check_index(q, w, k, pos, 4, 64, dtype=dtype)


# csa_index_scores: the scan alone, into caller rows; entries past the visible count untouched
@pytest.mark.parametrize("B,Q,E,H,d,dtype,m,lo,hi,e_cap_at", [
    (3, 1, 5000, 64, 128, "bf16", 4, 4 * 700, 4 * 5000, None),      # decode scan kernel
    (2, 1, 70000, 64, 128, "bf16", 4, 4 * 60000, 4 * 70000, None),  # rows past the segment size
    (1, 40, 3000, 64, 128, "bf16", 4, 4 * 3000 - 60, 4 * 3000, None),  # prefill scan kernel
    (2, 3, 700, 16, 64, "bf16", 4, 4 * 100, 4 * 700, 350),          # generic kernel, e_count
    (2, 2, 500, 4, 32, "f32", 1, -2, 500, None),                    # fp32, empty rows
])
def test_index_scores_call(B, Q, E, H, d, dtype, m, lo, hi, e_cap_at):
    q, w, k, pos = index_case(B, Q, E, H, d, dtype, lo, hi, m=m, seed=21)
    if B * Q > 1:
        pos.view(-1)[-1] = m * E - 1                  # one row sees every entry
    e_count = None
    if e_cap_at is not None:
        e_count = torch.full((B,), e_cap_at, dtype=torch.int32)
    sc = csa.IndexScores(dev(q), dev(w), dev(k), dev(pos), m, e_count=dev(e_count))
    sc.rows.fill_(float("nan"))                       # sentinel: must survive past n_vis
    got = sc().cpu().numpy()
    for b in range(B):
        for i in range(Q):
            t = int(pos[b, i])
            n_vis = ocsa.n_visible(t, m, E if e_count is None else int(e_count[b]))
            s = ocsa.index_scores(f64(q[b, i]), f64(w[b, i]), f64(k[b, :n_vis]))
            A = ocsa.score_scale(f64(q[b, i]), f64(w[b, i]), f64(k[b, :n_vis]))
            assert_scores(got[b, i, :n_vis], s, A, what=f"scores {(b, i)}")
            assert np.all(np.isnan(got[b, i, n_vis:])), f"row {(b, i)} written past n_vis"
    # the same kernel as inside csa_index_topk: its scores are bit-identical
    if H == 64 and d == 128 and e_count is None:
        _, alls = csa.index_topk(dev(q), dev(w), dev(k), dev(pos), m, 16, want_all=True)
        alls = alls.cpu().numpy()
        for b in range(B):
            for i in range(Q):
                n_vis = ocsa.n_visible(int(pos[b, i]), m, E)
                assert np.array_equal(got[b, i, :n_vis], alls[b, i, :n_vis])


def test_index_blocks_pool():
    B, E, bs, mb = 2, 6000, 8, 64
    q, w, k, pos = index_case(B, 1, E, 64, 128, "bf16", E - 5, E, m=1, seed=7)
    pos[1, 0] = 4001                         # partial last block
    # gap on block maxima at rank mb
    for b in range(B):
        n = ocsa.n_visible(int(pos[b, 0]), 1, E)
        R = ocsa.head_relu(f64(q[b, 0]), f64(k[b, :n]))
        attempt = 0
        while not gaps.gap_ok(ocsa.block_maxima(R @ f64(w[b, 0]), bs), mb):
            attempt += 1
            w[b, 0] = datagen.tensor(CID, 41, (64,), "bf16", 1 / 8, attempt, b).float()
    pool = csa.index_blocks(dev(q), dev(w), dev(k), dev(pos), 1, bs, mb, top_k=0).cpu()
    for b in range(B):
        ref_pool, s = pipeline.index_blocks_row(q[b, 0], w[b, 0], k[b], int(pos[b, 0]), 1, E, bs, mb)
        got = pool[b, 0].numpy()
        n = ref_pool.size
        assert_ids(got[:n], ref_pool, f"pool {b}")
        assert np.all(got[n:] == -1)


# ------------------------------------------------------------------------------ attention
def attn_case(B, Q, E, H, D, K, W, w_cap, dtype, seed=0, t_lo=None, t_hi=None):
    q = T(20, (B, Q, H, D), dtype, 1.0 if dtype == "f32" else 1 / math.sqrt(D), seed)
    kv = T(21, (B, E, D), dtype, 1.0 if dtype == "f32" else 1.0, seed)
    win = T(22, (B, w_cap, D), dtype, 1.0, seed)
    sink = T(23, (H,), "f32", 1.0, seed)
    g = np.random.default_rng(100 + seed)
    idx = np.full((B, Q, K), -1, np.int32)
    for b in range(B):
        for i in range(Q):
            n = int(g.integers(0, K + 1))
            idx[b, i, :n] = np.sort(g.choice(E, size=n, replace=False))
            g.shuffle(idx[b, i])
    lo = t_lo if t_lo is not None else 0
    hi = t_hi if t_hi is not None else 10 * w_cap
    pos = torch.from_numpy(g.integers(lo, hi, size=(B, Q)).astype(np.int64))
    return q, kv, torch.from_numpy(idx), win, sink, pos


def check_attn(q, kv, idx, win, sink, pos, w_cap, W, scale, dtype):
    out = csa.sparse_attn(dev(q), dev(kv), dev(idx), dev(win), w_cap, W, dev(pos), dev(sink),
                          scale).cpu()
    ref = pipeline.sparse_attn(q, kv, idx, win, w_cap, W, pos, sink, scale, dtype)
    for (b, i), r in ref.items():
        assert_rows_close(f64(out[b, i]), r, 2e-2, f"attn {(b, i)}")


@pytest.mark.parametrize("B,Q,E,K,W,w_cap", [
    (4, 1, 5000, 512, 128, 128),       # decode: row splits + combine
    (2, 3, 3000, 100, 128, 256),       # ragged tiles, ring larger than the window
    (1, 300, 2000, 512, 128, 4096),    # many rows: one workgroup per row
    (3, 1, 100, 0, 128, 128),          # window only
    (2, 2, 1000, 64, 0, 1),            # selection only
    (1, 256, 3000, 896, 128, 128),     # 32 tiles per row: the longest list held in LDS
    (1, 260, 4000, 2048, 128, 128),    # 68 tiles per row: register-staged tiles
    (1, 1, 5000, 2048, 128, 128),      # 68 one-tile splits: the combine's 64-partial round + one more
    (2, 1, 5000, 1536, 128, 128),      # 52 splits: the combine's 64-partial round alone
    (4, 1, 20000, 4096, 128, 128),     # 44 splits of 3 tiles: the double-buffered tile loop
])
def test_attention_fast_path(B, Q, E, K, W, w_cap):
    q, kv, idx, win, sink, pos = attn_case(B, Q, E, 64, 512, K, W, w_cap, "bf16",
                                           seed=B * 7 + Q, t_lo=0, t_hi=5 * w_cap)
    pos.view(-1)[0] = 5                # a window clamped at position 0
    check_attn(q, kv, idx, win, sink, pos, w_cap, W, 1 / math.sqrt(512), "bf16")


@pytest.mark.parametrize("B,Q", [(2, 1), (1, 260)])
def test_attention_sharp_logits(B, Q):
    # scaled queries make the softmax peaked: exercises the running-max rescale (one split of
    # 20 tiles per row when there are many rows)
    q, kv, idx, win, sink, pos = attn_case(B, Q, 3000, 64, 512, 512, 128, 128, "bf16", seed=9)
    q = (q.float() * 150).to(torch.bfloat16)
    check_attn(q, kv, idx, win, sink, pos, 128, 128, 1 / math.sqrt(512), "bf16")


def test_attention_no_sink_and_empty():
    q, kv, idx, win, sink, pos = attn_case(2, 1, 500, 64, 512, 64, 16, 16, "bf16", seed=10)
    idx[0, 0] = -1
    pos[0, 0] = -1                     # nothing at all: output 0
    out = csa.sparse_attn(dev(q), dev(kv), dev(idx), dev(win), 16, 16, dev(pos), None, 0.05).cpu()
    ref = pipeline.sparse_attn(q, kv, idx, win, 16, 16, pos, None, 0.05, "bf16")
    assert torch.all(out[0, 0] == 0)
    for (b, i), r in ref.items():
        assert_rows_close(f64(out[b, i]), r, 2e-2, f"attn {(b, i)}")


@pytest.mark.parametrize("H,D,dtype", [(4, 64, "f32"), (8, 128, "bf16"), (64, 512, "f32"),
                                       (3, 40, "f32")])
def test_attention_generic_path(H, D, dtype):
    q, kv, idx, win, sink, pos = attn_case(2, 3, 400, H, D, 64, 32, 64, dtype, seed=11)
    check_attn(q, kv, idx, win, sink, pos, 64, 32, 1 / math.sqrt(D), dtype)


# ------------------------------------------------------------------------------ MXFP4 keys
def _mx_tie_rows():
    """Rows of bf16-exact values that sit on the E2M1 rounding midpoints of their block."""
    from oracle import mx as omx
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 0.5, 6.0]
    rows = []
    for k in (-6, -3, 0, 4):
        r = np.zeros(128)
        for b in range(4):
            blk = np.array([(mids[(b + j) % len(mids)]) * (-1) ** j for j in range(32)])
            blk[0] = 6.0                       # block maximum 6 * 2^k -> scale 2^k
            r[32 * b:32 * b + 32] = blk * 2.0 ** k
        rows.append(r)
    rows.append(np.zeros(128))                 # zero blocks
    return np.array(rows)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_mxfp4_bit_exact(dtype):
    from oracle import mx as omx
    g = np.random.default_rng(31)
    x = g.standard_normal((300, 128)) / math.sqrt(128) * np.exp(0.5 * g.standard_normal((300, 1)))
    x = np.concatenate([x, _mx_tie_rows()])
    xt = torch.from_numpy(x).to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    codes, scales = csa.quantize_mxfp4(dev(xt))
    ref_c, ref_s = omx.quantize(f64(xt))
    assert np.array_equal(scales.cpu().numpy(), ref_s)
    assert np.array_equal(codes.cpu().numpy(), omx.pack(ref_c))


# ------------------------------------------------------------------------------ FP8 main cache
def _fp8_edge_rows():
    """Entries whose E4M3 channels sit on rounding midpoints (both signs), past the largest
    value, in the subnormal range, or at zero (all bf16-exact)."""
    from oracle import fp8 as of8
    fin = of8.E4M3_VALUES[np.isfinite(of8.E4M3_VALUES)]
    mag = np.sort(np.unique(np.abs(fin)))
    special = np.concatenate([(mag[1:] + mag[:-1]) / 2, [464.0, 500.0, 1e4, 2.0 ** -10,
                                                         3 * 2.0 ** -11, 2.0 ** -12, 0.0]])
    rows = []
    for sign in (1.0, -1.0):
        r = np.resize(special * sign, 512)
        r[448:] = np.linspace(-3, 3, 64)
        rows.append(r)
    return np.array(rows)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_kv_fp8_bit_exact(dtype):
    from oracle import fp8 as of8
    g = np.random.default_rng(41)
    x = g.standard_normal((200, 512)) * np.exp(0.7 * g.standard_normal((200, 1)))
    x = np.concatenate([x, _fp8_edge_rows()])
    xt = torch.from_numpy(x).to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    got = csa.quantize_kv_fp8(dev(xt)).cpu().numpy()
    want = of8.encode_entries(f64(xt))
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"first mismatch at {tuple(bad[0])}: {got[tuple(bad[0])]} vs {want[tuple(bad[0])]}"


def test_dequantize_kv_fp8_every_code():
    """Every finite E4M3 code decodes to its exact value (hardware conversion, scale 1); the
    rotary channels pass through."""
    from oracle import fp8 as of8
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    e = np.zeros((3, 576), np.uint8)
    for r in range(3):
        e[r, :448] = np.resize(np.roll(codes, 97 * r), 448)
        e[r, 448:] = np.random.default_rng(r).integers(0, 256, 128).astype(np.uint8)
        e[r, 449::2] &= 0x3F   # finite bf16 rotary values (top exponent bit clear)
    out = csa.dequantize_kv_fp8(dev(torch.from_numpy(e))).cpu()
    np.testing.assert_array_equal(f64(out), of8.decode_entries(e))


@pytest.mark.parametrize("B,Q,E,K,W,w_cap", [
    (4, 1, 5000, 512, 128, 128),       # decode: row splits + combine
    (2, 3, 3000, 100, 128, 256),       # ragged tiles: FP8 and window rows share a tile
    (1, 300, 2000, 512, 128, 4096),    # many rows: one workgroup per row
    (2, 2, 1000, 64, 0, 1),            # selection only
    (1, 256, 3000, 896, 128, 128),     # 32 tiles per row: the longest list held in LDS
    (1, 260, 4000, 2048, 128, 128),    # 68 tiles per row: register-staged tiles
])
def test_attention_fp8_cache(B, Q, E, K, W, w_cap):
    """csa_sparse_attn_fp8 against the oracle's attention over the entries' FP8 values."""
    from oracle import fp8 as of8
    q, kv, idx, win, sink, pos = attn_case(B, Q, E, 64, 512, K, W, w_cap, "bf16",
                                           seed=B * 11 + Q, t_lo=0, t_hi=5 * w_cap)
    pos.view(-1)[0] = 5
    k8 = csa.quantize_kv_fp8(dev(kv))
    enc = of8.encode_entries(f64(kv))
    assert np.array_equal(k8.cpu().numpy(), enc)
    scale = 1 / math.sqrt(512)
    out = csa.sparse_attn(dev(q), k8, dev(idx), dev(win), w_cap, W, dev(pos), dev(sink),
                          scale).cpu()
    kv_vals = torch.from_numpy(of8.decode_entries(enc))
    ref = pipeline.sparse_attn(q, kv_vals, idx, win, w_cap, W, pos, sink, scale, "bf16")
    for (b, i), r in ref.items():
        assert_rows_close(f64(out[b, i]), r, 2e-2, f"attn fp8 {(b, i)}")


# ------------------------------------------------------------------------------ FP4 main cache
def _fp4_edge_rows():
    """Entries whose blocks put amax / 6 on an E4M3 rounding midpoint (a tie of the scale), or
    their elements on E2M1 midpoints times the scale (ties of the codes), both signs; blocks past
    the largest scale, at the zero-scale tie and just above it, zero blocks and negative zeros
    (every value bf16-exact)."""
    from oracle import fp8 as of8
    mags = np.sort(np.unique(np.abs(of8.E4M3_VALUES[np.isfinite(of8.E4M3_VALUES)])))
    s_mids = (mags[1:] + mags[:-1]) / 2                  # amax / 6 on a scale tie
    e_mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    blocks = []
    for k, sm in enumerate(s_mids[::3]):
        b = np.zeros(16)
        b[0] = 6 * sm * (-1) ** k
        blocks.append(b)
    for k, sv in enumerate([1.0, 1.125, 0.875 * 2.0 ** -4, 1.5 * 2.0 ** 3, 2.0 ** -9, 448.0]):
        b = np.zeros(16)
        b[0] = 6 * sv                                    # amax / 6 = sv exactly
        b[1:8] = e_mids * sv
        b[8:15] = -e_mids * sv
        blocks.append(b)
    for amax in (2688.0, 3072.0, 16384.0, 6 * 2.0 ** -10, 6.25 * 2.0 ** -10, 0.0):
        b = amax * np.arange(-8, 8) / 8                  # bf16-exact steps
        b[0] = -amax
        blocks.append(b)
    b = np.zeros(16)
    b[0], b[1] = 1.0, -0.0
    blocks.append(b)
    flat = np.concatenate(blocks)
    rows = np.resize(flat, (int(np.ceil(flat.size / 512)), 512))
    return np.concatenate([rows, -rows])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_kv_fp4_bit_exact(dtype):
    from oracle import kv_fp4 as of4
    g = np.random.default_rng(45)
    x = g.standard_normal((200, 512)) * np.exp(0.7 * g.standard_normal((200, 1)))
    x[5] *= 1e-3                                           # small scales, subnormal ones
    x[6] *= 1e3                                            # saturating scales
    x = np.concatenate([x, _fp4_edge_rows()])
    xt = torch.from_numpy(x).to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    if dtype == "f32":   # one fp32 ulp either side of every value of the edge rows
        e = torch.from_numpy(_fp4_edge_rows()).float()
        xt = torch.cat([xt, torch.nextafter(e, torch.full_like(e, np.inf)),
                        torch.nextafter(e, torch.full_like(e, -np.inf))])
    got = csa.quantize_kv_fp4(dev(xt)).cpu().numpy()
    want = of4.encode_entries(f64(xt))
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"first mismatch at {tuple(bad[0])}: {got[tuple(bad[0])]} vs {want[tuple(bad[0])]}"


def test_dequantize_kv_fp4_every_code_and_scale():
    """Every E2M1 code under every finite E4M3 scale code decodes to element x scale exactly."""
    from oracle import kv_fp4 as of4
    scales = np.arange(0, 0x7F, dtype=np.uint8)           # 0 .. 448
    e = np.zeros((len(scales), 288), np.uint8)
    g = np.random.default_rng(46)
    for r, sc in enumerate(scales):
        e[r, :256] = np.resize(np.arange(256, dtype=np.uint8), 256)   # every code pair
        e[r, 256:] = np.roll(scales, r)[:32]
        e[r, 256 + r % 32] = sc
    e[:, :256] = np.where(g.random((len(scales), 256)) < 0.1, 0x88, e[:, :256])  # -0 codes
    out = csa.dequantize_kv_fp4(dev(torch.from_numpy(e))).cpu()
    np.testing.assert_array_equal(f64(out), of4.decode_entries(e))


@pytest.mark.parametrize("B,Q,E,K,W,w_cap", [
    (4, 1, 5000, 512, 128, 128),       # decode: row splits + combine
    (2, 3, 3000, 100, 128, 256),       # ragged tiles: FP4 and window rows share a tile
    (1, 300, 2000, 512, 128, 4096),    # many rows: one workgroup per row
    (2, 2, 1000, 64, 0, 1),            # selection only
    (1, 256, 3000, 896, 128, 128),     # 32 tiles per row: the longest list held in LDS
    (1, 260, 4000, 2048, 128, 128),    # 68 tiles per row: register-staged tiles
])
def test_attention_fp4_cache(B, Q, E, K, W, w_cap):
    """csa_sparse_attn_fp4 against the oracle's attention over the entries' FP4 values."""
    from oracle import kv_fp4 as of4
    q, kv, idx, win, sink, pos = attn_case(B, Q, E, 64, 512, K, W, w_cap, "bf16",
                                           seed=B * 13 + Q, t_lo=0, t_hi=5 * w_cap)
    pos.view(-1)[0] = 5
    k4 = csa.quantize_kv_fp4(dev(kv))
    enc = of4.encode_entries(f64(kv))
    assert np.array_equal(k4.cpu().numpy(), enc)
    scale = 1 / math.sqrt(512)
    out = csa.sparse_attn(dev(q), k4, dev(idx), dev(win), w_cap, W, dev(pos), dev(sink),
                          scale).cpu()
    kv_vals = torch.from_numpy(of4.decode_entries(enc))
    ref = pipeline.sparse_attn(q, kv_vals, idx, win, w_cap, W, pos, sink, scale, "bf16")
    for (b, i), r in ref.items():
        assert_rows_close(f64(out[b, i]), r, 2e-2, f"attn fp4 {(b, i)}")


def test_bf16_rounding_of_fp32_values():
    """The fp32 -> bf16 rounding every kernel stores with (here through the FP8 entry's 64
    bf16 channels of an fp32 input) is round-to-nearest-even on the bit pattern: exact ties
    of both parities, the values one fp32 ulp either side of a tie, fp32 subnormals, the
    largest finite values (rounding past the bf16 maximum gives inf) and signed zeros
    against the oracle's rounding."""
    from oracle import fp8 as of8
    g = np.random.default_rng(43)
    base = g.standard_normal(4096).astype(np.float32) * np.float32(2.0) ** g.integers(
        -60, 60, 4096).astype(np.float32)
    b = base.view(np.uint32) & np.uint32(0xffff0000)              # bf16-exact values
    tie = (b | np.uint32(0x8000)).view(np.float32)                # halfway to the next one
    vals = np.concatenate([
        tie, (tie.view(np.uint32) - 1).view(np.float32), (tie.view(np.uint32) + 1).view(np.float32),
        np.array([1e-39, -1e-39, 2.0 ** -130, 3 * 2.0 ** -134, 2.0 ** -149, 1.1754942e-38,
                  3.3895314e38, -3.3895314e38, 3.4028235e38, 3.3961776e38, 0.0, -0.0],
                 dtype=np.float32)])
    n = (vals.size + 63) // 64
    x = np.zeros((n, 512), np.float32)
    x[:, 448:].flat[:vals.size] = vals
    xt = torch.from_numpy(x)
    got = csa.quantize_kv_fp8(dev(xt)).cpu().numpy()
    want = of8.encode_entries(f64(xt))
    bad = np.argwhere(got[:, 448:] != want[:, 448:])
    assert bad.size == 0, f"first mismatch at {tuple(bad[0])}"
