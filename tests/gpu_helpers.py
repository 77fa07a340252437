"""Shared helpers of the GPU parity tests (inputs from datagen, expectations from the oracle)."""
import math

import numpy as np
import torch

import datagen
import sparse_long_context_csa_amd as csa_lib
from oracle import csa as ocsa
from oracle import fp8, gaps, kv_fp4, mx
from oracle.pipeline import f64, i64

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
T_TEST_W = 40


def dev(t):
    return t.to(DEV) if isinstance(t, torch.Tensor) else t


def fix_gaps(case_id, q_idx, w, k_idx, q_pos, e_count, m, K, cand=None, dtype="bf16"):
    """Redraw gate rows (seeded) until each row's visible scores separate at rank K."""
    B, Q, H, _ = q_idx.shape
    qp = i64(q_pos)
    E = k_idx.shape[1]
    ec = i64(e_count) if e_count is not None else np.full(B, E)
    for b in range(B):
        keys = f64(k_idx[b])
        for i in range(Q):
            n = ocsa.n_visible(int(qp[b, i]), m, int(min(ec[b], E)))
            ids = np.arange(n)
            if cand is not None:
                c = i64(cand[b, i])
                ids = c[(c >= 0) & (c < n)]
            R = ocsa.head_relu(f64(q_idx[b, i]), keys[ids])
            attempt = 0
            while not gaps.gap_ok(R @ f64(w[b, i]), K):
                attempt += 1
                assert attempt < 5000
                w[b, i] = datagen.tensor(case_id, T_TEST_W, (H,), dtype, 1 / math.sqrt(H), attempt,
                                         b, i).float()


def assert_ids(gpu, ref, what=""):
    g = np.asarray(gpu, dtype=np.int64)
    r = np.asarray(ref, dtype=np.int64)
    if not np.array_equal(g, r):
        bad = np.argwhere(g != r)
        raise AssertionError(f"{what}: ids differ at {bad[:5].tolist()} "
                             f"(gpu {g[tuple(bad[0])]}, oracle {r[tuple(bad[0])]})")


def assert_scores(gpu, ref, scale, rel=1e-3, what=""):
    """|S_gpu - S_ref| <= rel * A + tiny, A = sum_h |w| relu(q.k)."""
    g = np.asarray(gpu, dtype=np.float64)
    err = np.abs(g - ref)
    tol = rel * scale + 1e-30
    if not np.all(err <= tol):
        k = int(np.argmax(err / tol))
        raise AssertionError(f"{what}: score error {err[k]:.3e} > {tol[k]:.3e} at {k}")


def assert_rows_close(gpu, ref, rel=2e-2, what=""):
    """Per (query, head) row: max|diff| <= rel * max|ref| (rows of ref that are all zero must be
    zero on the GPU up to 1e-30)."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    err = np.abs(g - r).max(axis=-1)
    den = np.abs(r).max(axis=-1)
    ok = err <= rel * den + 1e-30
    if not np.all(ok):
        k = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: row {k.tolist()} error {err[tuple(k)]:.3e} vs "
                             f"max|ref| {den[tuple(k)]:.3e}")


def bf16_ulp(x):
    """The spacing of bf16 values at |x| (normal range)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.maximum(x, 2.0 ** -126))
    return np.ldexp(1.0, e - 8)


def assert_pooled(got, exact, xabs_max, what="", m=16):
    """A pooled entry computed in fp32 and stored once by RNE: |got - exact| is at most half a
    storage spacing at max(|got|, |exact|) plus the fp32 arithmetic error, bounded by
    (m + 8) * 2^-24 * max_j |x_j| (<= 4e-6 * max_j |x_j| for m <= 16; pooling over more rows
    passes its m)."""
    got = np.asarray(got, dtype=np.float64)
    exact = np.asarray(exact, dtype=np.float64)
    slack = max(4e-6, 2.0 * (m + 8) * 2.0 ** -24)
    tol = 0.5 * bf16_ulp(np.maximum(np.abs(got), np.abs(exact))) + slack * np.asarray(xabs_max)
    bad = np.abs(got - exact) > tol
    if np.any(bad):
        k = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: pooled value {got[k]} vs exact {exact[k]} (tol {tol[k]:.3e})")


def assert_mx_entry(codes, scales, exact, xabs_max, what=""):
    """The MXFP4 form of a pooled key. The oracle's cached key is quantise(round_bf16(exact));
    the GPU rounds its fp32 pooling to bf16, which can land on the other bf16 neighbour only
    where exact lies within the fp32 error (4e-6 max_j |x_j|) of a rounding midpoint. Blocks
    without such an element must match the oracle's codes and scale byte exactly; the others
    must hold a valid MXFP4 rounding of a value within that error: off by at most half an E2M1
    gap (at most 2^s) or, for magnitudes past 6 x 2^s, by the saturation to 6 x 2^s, plus one
    bf16 spacing."""
    kb = ocsa.store(exact, "bf16")
    tol = 4e-6 * np.asarray(xabs_max)
    near_mid = np.abs(exact - kb) >= 0.5 * bf16_ulp(kb) - tol
    oc, osc = mx.quantize(kb)
    gc = mx.unpack(np.asarray(codes, dtype=np.uint8))
    gs = np.asarray(scales, dtype=np.uint8)
    deq = mx.dequantize(gc, gs)
    for blk in range(gs.size):
        sl = slice(32 * blk, 32 * blk + 32)
        if not near_mid[sl].any():
            assert gs[blk] == osc[blk] and np.array_equal(gc[sl], oc[sl]), \
                f"{what}: block {blk} codes/scale differ from the oracle's"
            continue
        step = 2.0 ** (float(gs[blk]) - 127)
        assert abs(int(gs[blk]) - int(osc[blk])) <= 1, f"{what}: block {blk} scale"
        err = np.abs(deq[sl] - exact[sl])
        bound = np.maximum(step, np.abs(exact[sl]) - 6 * step)
        assert np.all(err <= bound + bf16_ulp(kb[sl]) + tol[sl]), f"{what}: block {blk} values"


def pooled_xmax(x, m):
    """max_j |x[e*m + j, c]| per (entry, channel) of rows x [..., T, d]."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    sh = a.shape
    return a.reshape(sh[:-2] + (sh[-2] // m, m, sh[-1])).max(axis=-2)


def mxfp4_case(spec):
    """A decode case with an MXFP4 indexer cache. The oracle's case holds the MXFP4 values of
    the generated bf16 keys (oracle quantiser); the GPU gets the codes and scale bytes that
    csa_quantize_mxfp4 makes of the same bf16 keys (returned, on the device)."""
    case = datagen.make_case(spec)
    k = case["k_idx"]
    codes, scales = mx.quantize(f64(k))
    case["k_idx"] = torch.from_numpy(mx.dequantize(codes, scales)).to(k.dtype)
    case["idx_format"] = "mxfp4"
    kc, ks = csa_lib.quantize_mxfp4(dev(k))
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), mx.pack(codes))
    assert np.array_equal(ks.cpu().numpy(), scales)
    return case, {"k_idx": kc, "k_idx_scale": ks}


def assert_fp8_entry(entry, exact, xabs_max, what=""):
    """The FP8 form of a pooled main entry. The GPU's fp32 pooling lies within 4e-6 max_j |x_j|
    of the exact value; rounding to bf16 and then to E4M3 (or bf16 for the rotary channels) is
    monotone, so each stored value lies between the cached values of exact -/+ that error (the
    same value, hence bit-exact, wherever no rounding boundary falls in between)."""
    tol = 4e-6 * np.asarray(xabs_max)
    lo = fp8.cached_entries(ocsa.store(exact - tol, "bf16"))
    hi = fp8.cached_entries(ocsa.store(exact + tol, "bf16"))
    got = fp8.decode_entries(np.asarray(entry, dtype=np.uint8))
    bad = (got < lo) | (got > hi)
    if np.any(bad):
        k = int(np.argwhere(bad)[0][0])
        raise AssertionError(f"{what}: channel {k} holds {got[k]}, outside [{lo[k]}, {hi[k]}] "
                             f"(exact {exact[k]})")


def assert_fp4_entry(entry, exact, xabs_max, what=""):
    """The FP4 form of a pooled main entry. The GPU's fp32 pooling lies within 4e-6 max_j |x_j|
    of the exact value, and the stored bf16 value between the roundings of exact -/+ that error.
    A block's scale is monotone in its largest magnitude, so the stored scale code lies between
    those of the smallest and largest possible maxima; under the scale the GPU chose, each
    element's cached value is monotone in the element, so it lies between the cached values of
    the two bounds (bit-exact wherever no rounding boundary falls in between)."""
    tol = 4e-6 * np.asarray(xabs_max)
    lo = ocsa.store(exact - tol, "bf16")
    hi = ocsa.store(exact + tol, "bf16")
    e = np.asarray(entry, dtype=np.uint8)
    sc = e[kv_fp4.CODE_BYTES:].astype(np.int64)
    mag_hi = np.maximum(np.abs(lo), np.abs(hi)).reshape(32, 16).max(axis=1)
    mag_lo = np.where(np.sign(lo) == np.sign(hi), np.minimum(np.abs(lo), np.abs(hi)), 0.0)
    mag_lo = mag_lo.reshape(32, 16).max(axis=1)
    sc_lo = kv_fp4.block_scale_codes(mag_lo).astype(np.int64)
    sc_hi = kv_fp4.block_scale_codes(mag_hi).astype(np.int64)
    bad = np.flatnonzero((sc < sc_lo) | (sc > sc_hi))
    if bad.size:
        g = int(bad[0])
        raise AssertionError(f"{what}: block {g} scale code {sc[g]} outside [{sc_lo[g]}, "
                             f"{sc_hi[g]}]")
    s = np.repeat(fp8.dequantize(sc.astype(np.uint8)), 16)
    got = kv_fp4.decode_entries(e)

    def cached(v):
        y = np.divide(v, s, out=np.zeros_like(v), where=s > 0)
        return kv_fp4.E2M1_VALUES[kv_fp4.nearest_e2m1(y)] * s

    clo, chi = cached(lo), cached(hi)
    bad = np.flatnonzero((got < clo) | (got > chi))
    if bad.size:
        k = int(bad[0])
        raise AssertionError(f"{what}: channel {k} holds {got[k]}, outside [{clo[k]}, {chi[k]}] "
                             f"(exact {exact[k]})")


def fp4_case(case):
    """fp8_case for an FP4 main cache (288-byte entries, csa_quantize_kv_fp4 against the oracle's
    encoder). Returns the device state {"kv": uint8 [B, E, 288]}."""
    kv = case["kv"]
    want = kv_fp4.encode_entries(f64(kv))
    case["kv"] = torch.from_numpy(kv_fp4.decode_entries(want)).to(kv.dtype)
    case["kv_format"] = "fp4"
    k4 = csa_lib.quantize_kv_fp4(dev(kv))
    torch.cuda.synchronize()
    assert np.array_equal(k4.cpu().numpy(), want)
    return {"kv": k4}


def quant_case(case, fmt):
    """The device state of a main cache in fmt ("fp8" or "fp4"), the case updated to match."""
    return fp8_case(case) if fmt == "fp8" else fp4_case(case)


def fp8_case(case):
    """Turns a bf16 decode case into one with an FP8 main cache: the oracle's case holds the
    cached values of the generated entries (oracle encoder); the GPU gets the entries that
    csa_quantize_kv_fp8 makes of the same bf16 values, checked equal byte for byte. Returns
    the device state {"kv": uint8 [B, E, 576]}."""
    kv = case["kv"]
    want = fp8.encode_entries(f64(kv))
    case["kv"] = torch.from_numpy(fp8.decode_entries(want)).to(kv.dtype)
    case["kv_format"] = "fp8"
    k8 = csa_lib.quantize_kv_fp8(dev(kv))
    torch.cuda.synchronize()
    assert np.array_equal(k8.cpu().numpy(), want)
    return {"kv": k8}


def run_step(case, idx_state=None):
    """One csa_decode_step over copies of the case's state (idx_state: device tensors that
    replace the case's own, e.g. the MXFP4 indexer cache {"k_idx": codes, "k_idx_scale":
    scales} or the FP8 main cache {"kv": entries})."""
    spec = case["spec"]
    g = {k: dev(v) for k, v in case.items() if isinstance(v, torch.Tensor)}
    rings = [dev(r).clone() for r in case["rings"]]
    win_new = [g["x_new"] if (c == 0 and datagen.ring_from_raw(spec)) else None
               for c in range(spec.n_attn)]
    kw = {}
    if spec.block_size:
        kw = dict(block_size=spec.block_size, max_blocks=spec.max_blocks, q_idx2=g["q_idx2"],
                  w2=g["w2"])
    names = ["kv", "k_idx", "x_tail", "z_tail", "xi_tail", "zi_tail"]
    c4a = case.get("compressor") == "c4a"
    if c4a:
        names += ["xb_tail", "zb_tail"]
        kw.update(compressor="c4a", xb_new=g["xb_new"], zb_new=g["zb_new"], bias_b=g["bias_b"])
    st = {k: g[k].clone() for k in names}
    if idx_state is not None:
        st.update({k: v.clone() for k, v in idx_state.items()})
    step = csa_lib.DecodeStep(m=spec.m, top_k=spec.K, window=spec.W, scale=case["scale"],
                          pos=g["pos"], x_new=g["x_new"], z_new=g["z_new"], xi_new=g["xi_new"],
                          zi_new=g["zi_new"], bias=g["bias"], bias_i=g["bias_i"],
                          q_idx=g["q_idx"], w=g["w"], q=[dev(x) for x in case["q"]], win=rings,
                          win_new=win_new, sink=[dev(x) for x in case["sink"]],
                          score_format=case.get("score_format", "f32"),
                          out_rope_dim=int(case.get("out_rope_dim", 0)),
                          q_gamma=[dev(x) if x is not None else None
                                   for x in (case.get("q_gamma") or [])],
                          q_rope_dim=int(case.get("q_rope_dim", 0)),
                          kv_gamma=(dev(case["kv_gamma"]) if case.get("kv_gamma") is not None
                                    else None),
                          kv_rope_dim=int(case.get("kv_rope_dim", 0)),
                          query_fp4=case.get("idx_format") == "mxfp4_qk", **st, **kw)
    out, idx = step()
    torch.cuda.synchronize()
    return step, st, rings, [o.cpu() for o in out], idx.cpu()


def check_step(case, ref, st, rings, out, idx):
    spec = case["spec"]
    for b in range(spec.B):
        t = int(case["pos"][b])
        assert_ids(idx[b].numpy(), ref["ids"][b], f"seq {b}")
        for c in range(spec.n_attn):
            assert_rows_close(f64(out[c][b]), ref["out"][b][c], 2e-2, f"seq {b} call {c}")
        slot = t % spec.m
        assert torch.equal(st["x_tail"][b, slot].cpu(), case["x_new"][b])
        assert torch.equal(st["zi_tail"][b, slot].cpu(), case["zi_new"][b])
        c4a = case.get("compressor") == "c4a"
        if c4a:   # the b stream's new row in its two-block ring; the other rows untouched
            rb = t % (2 * spec.m)
            keep = np.arange(2 * spec.m) != rb
            for name, new in (("xb_tail", "xb_new"), ("zb_tail", "zb_new")):
                got = st[name][b].cpu()
                assert torch.equal(got[rb], case[new][b])
                assert torch.equal(got[keep], case[name][b][keep])
        if b in ref["kv_new"]:
            e = (t + 1) // spec.m - 1
            for name, xs, zs, xn, zn, bias in (
                    ("kv", "x_tail", "z_tail", "x_new", "z_new", "bias"),
                    ("k_idx", "xi_tail", "zi_tail", "xi_new", "zi_new", "bias_i")):
                x = f64(case[xs][b]).copy()
                z = f64(case[zs][b]).copy()
                x[slot] = f64(case[xn][b])
                z[slot] = f64(case[zn][b])
                exact = ocsa.compress(x, z, f64(case[bias]), spec.m)[0]
                xmax = np.abs(x).max(axis=0)
                if name == "kv" and c4a:
                    # the overlapped entry (oracle), over this block's a rows and the b rows
                    # of the block before
                    exact = ref["kv_new_exact"][b]
                    rows = [x]
                    if e > 0:
                        h = ((e - 1) % 2) * spec.m
                        rows.append(f64(case["xb_tail"][b])[h:h + spec.m])
                    xmax = np.abs(np.concatenate(rows)).max(axis=0)
                if name == "kv" and b in ref.get("kv_new_exact", {}) and (
                        case.get("kv_gamma") is not None or case.get("kv_rope_dim")):
                    # normalised / rotated: the fp32 error scales with the entry itself
                    exact = ref["kv_new_exact"][b]
                    xmax = np.full(exact.shape, 4.0 * np.abs(exact).max())
                if name == "kv" and case.get("kv_format") == "fp8":
                    assert_fp8_entry(st["kv"][b, e].cpu().numpy(), exact, xmax,
                                     f"FP8 entry {e} of seq {b}")
                    continue
                if name == "kv" and case.get("kv_format") == "fp4":
                    assert_fp4_entry(st["kv"][b, e].cpu().numpy(), exact, xmax,
                                     f"FP4 entry {e} of seq {b}")
                    continue
                if name == "k_idx" and case.get("idx_format") in ("mxfp4", "mxfp4_qk"):
                    assert_mx_entry(st["k_idx"][b, e].cpu().numpy(),
                                    st["k_idx_scale"][b, e].cpu().numpy(), exact,
                                    np.abs(x).max(axis=0), f"MXFP4 key entry {e} of seq {b}")
                    continue
                assert_pooled(f64(st[name][b, e].cpu()), exact, xmax,
                              f"{name} entry {e} of seq {b}")
        if datagen.ring_from_raw(spec):
            got = rings[0][b, t % spec.w_cap].cpu()
            if b in ref.get("win_row_exact", {}):
                # the new window row, normalised and rotated at t like an entry
                exact = ref["win_row_exact"][b]
                assert_pooled(f64(got), exact, np.full(exact.shape, 4.0 * np.abs(exact).max()),
                              f"window row {t} of seq {b}")
            else:
                assert torch.equal(got, case["x_new"][b])


