"""Pins of the oracle drivers: the decode step, the prefill chunk and the tiny forward are
compositions of the pinned primitives; causality and reduction invariants hold."""
import numpy as np
import pytest
import torch

import datagen
from oracle import csa, fp8, gaps, kv_fp4, mx, pipeline
from oracle.pipeline import f64


def small_decode(**kw):
    base = dict(case_id=901, kind="decode", B=3, L=4096, m=4, H_I=8, d_I=16, H=4, D=32,
                K=16, W=8, w_cap=16, ragged=True)
    base.update(kw)
    return datagen.make_case(datagen.CaseSpec(**base))


def test_decode_step_new_entry_is_pooled_tail():
    case = small_decode()
    res = pipeline.decode_step(case)
    spec = case["spec"]
    for b in range(spec.B):
        t = int(case["pos"][b])
        if (t + 1) % spec.m:
            assert b not in res["kv_new"]
            continue
        x = f64(case["x_tail"][b]).copy()
        z = f64(case["z_tail"][b]).copy()
        x[t % spec.m] = f64(case["x_new"][b])
        z[t % spec.m] = f64(case["z_new"][b])
        np.testing.assert_array_equal(
            res["kv_new"][b], csa.round_bf16(csa.compress(x, z, f64(case["bias"]), spec.m)[0]))


def test_decode_positions_cover_block_phases():
    case = small_decode(B=8)
    phases = {int(t) % 4 for t in case["pos"]}
    assert len(phases) > 1 and 3 in phases     # seq 0 sits at L-1: block completes


def test_decode_step_is_the_composition_of_primitives():
    case = small_decode()
    spec = case["spec"]
    res = pipeline.decode_step(case)
    for b in range(spec.B):
        t = int(case["pos"][b])
        n = csa.n_visible(t, spec.m, spec.entries)
        keys = f64(case["k_idx"][b][:n]).copy()
        kv = f64(case["kv"][b]).copy()
        if b in res["ki_new"]:
            e = (t + 1) // spec.m - 1
            keys[e] = res["ki_new"][b]
            kv[e] = res["kv_new"][b]
        ids = csa.select_topk(csa.index_scores(f64(case["q_idx"][b]), f64(case["w"][b]), keys), spec.K)
        assert res["ids"][b].tolist() == ids.tolist()
        ring = f64(case["rings"][0][b]).copy()
        ring[t % spec.w_cap] = f64(case["x_new"][b])
        o = csa.sink_attention(f64(case["q"][0][b]),
                               csa.attention_rows(kv, ids, ring, spec.w_cap, spec.W, t),
                               f64(case["sink"][0]), case["scale"])
        np.testing.assert_array_equal(res["out"][b][0], csa.round_bf16(o))


def test_decode_step_ignores_invisible_entries_and_old_ring_rows():
    case = small_decode()
    spec = case["spec"]
    base = pipeline.decode_step(case)
    case2 = dict(case)
    kv, ki = case["kv"].clone(), case["k_idx"].clone()
    ring = case["rings"][0].clone()
    for b in range(spec.B):
        t = int(case["pos"][b])
        n = csa.n_visible(t, spec.m, spec.entries)
        e_new = (t + 1) // spec.m - 1 if (t + 1) % spec.m == 0 else n
        kv[b, n:] = 50.0
        ki[b, n:] = 50.0
        if e_new < n:                      # the entry being completed is recomputed
            kv[b, e_new] = -50.0
            ki[b, e_new] = -50.0
        for p in range(t - spec.w_cap + 1, t - spec.W + 1):
            ring[b, p % spec.w_cap] = 77.0
    case2.update(kv=kv, k_idx=ki, rings=[ring])
    res = pipeline.decode_step(case2)
    for b in range(spec.B):
        assert res["ids"][b].tolist() == base["ids"][b].tolist()
        np.testing.assert_array_equal(res["out"][b][0], base["out"][b][0])


def test_hierarchical_with_full_budget_is_flat_with_second_query():
    case = small_decode(case_id=902, m=1, L=300, block_size=4, max_blocks=100, n_attn=2,
                        ragged=False)
    spec = case["spec"]
    res = pipeline.decode_step(case)
    for b in range(spec.B):
        n = res["n_vis"][b]
        assert res["pool"][b].tolist() == list(range(n))
        keys = f64(case["k_idx"][b][:n]).copy()
        keys[n - 1] = res["ki_new"][b]
        flat = csa.select_topk(csa.index_scores(f64(case["q_idx2"][b]), f64(case["w2"][b]), keys), spec.K)
        assert res["ids"][b].tolist() == flat.tolist()
        assert len(res["out"][b]) == 2


def test_hierarchical_pool_is_budgeted():
    case = small_decode(case_id=903, m=1, L=600, block_size=4, max_blocks=10, ragged=False)
    res = pipeline.decode_step(case)
    for b, pool in res["pool"].items():
        assert pool.size == 40
        assert set(res["ids"][b][res["ids"][b] >= 0].tolist()) <= set(pool.tolist())


def test_m1_new_entry_is_the_raw_row():
    case = small_decode(case_id=904, m=1, L=100, ragged=False)
    res = pipeline.decode_step(case)
    for b in range(case["spec"].B):
        np.testing.assert_array_equal(res["kv_new"][b], f64(case["x_new"][b]))
        np.testing.assert_array_equal(res["ki_new"][b], f64(case["xi_new"][b]))


def test_fp4_query_key_path_hand_worked():
    # [CoD "FP4, down to the index scores"]: the query-key path multiplies FP4 values. One head,
    # one 32-channel block of the query: max |q| = 0.75 -> s = -3, q / 2^s = 8 q rounds to
    # [6, 1, 1.5, 0, 1, -2, 1, 2, 4, -6] (ties to the even code), i.e. q4 = [0.75, 0.125,
    # 0.1875, 0, 0.125, -0.25, 0.125, 0.25, 0.5, -0.75]; a key of ones is exact in MXFP4. Score
    # w * ReLU(q4 . k) = 1.0625 against 1.03125 for the unquantised query.
    q = np.zeros((1, 32))
    q[0, :10] = [0.75, 0.1, 0.2, 0.03125, 0.09375, -0.3, 0.15625, 0.3125, 0.4375, -0.75]
    case = {"idx_format": "mxfp4_qk"}
    q4 = pipeline.index_query(case, q)
    assert q4[0, :10].tolist() == [0.75, 0.125, 0.1875, 0.0, 0.125, -0.25, 0.125, 0.25, 0.5,
                                   -0.75]
    k = pipeline.cached_index_key(case, np.ones(32))
    assert np.array_equal(k, np.ones(32))
    assert csa.index_scores(q4, np.ones(1), k[None])[0] == 1.0625
    assert csa.index_scores(pipeline.index_query({"idx_format": "mxfp4"}, q), np.ones(1),
                            k[None])[0] == 1.03125


def test_fp4_query_key_path_quantises_each_head():
    # the decode step on the FP4 query-key path equals the MXFP4-key step given, for each head
    # on its own, the query's MXFP4 value (quantised here block by block in a loop); its scores
    # differ from those of the bf16 query
    case = small_decode(case_id=907, m=1, L=300, d_I=64, ragged=False)
    spec = case["spec"]
    res = pipeline.decode_step(dict(case, idx_format="mxfp4_qk"))
    qv = f64(case["q_idx"]).copy()
    for b in range(spec.B):
        for h in range(spec.H_I):
            for blk in range(spec.d_I // 32):
                v = qv[b, h, 32 * blk:32 * blk + 32]
                c, sc = mx.quantize(v[None])
                qv[b, h, 32 * blk:32 * blk + 32] = mx.dequantize(c, sc)[0]
    moved = dict(case, idx_format="mxfp4", q_idx=torch.from_numpy(qv))
    want = pipeline.decode_step(moved)
    plain = pipeline.decode_step(dict(case, idx_format="mxfp4"))
    for b in range(spec.B):
        np.testing.assert_array_equal(res["scores"][b], want["scores"][b])
        np.testing.assert_array_equal(res["ids"][b], want["ids"][b])
        assert not np.array_equal(res["scores"][b], plain["scores"][b])


def test_mxfp4_cache_scores_the_new_key_on_the_grid():
    # m = 1: the new entry's key is the raw row xi_new; with an MXFP4 cache it is scored at its
    # E2M1 x 2^s value, every other entry as case["k_idx"] holds it
    case = small_decode(case_id=905, m=1, L=300, d_I=64, ragged=False)
    spec = case["spec"]
    bf = pipeline.decode_step(case)
    case["idx_format"] = "mxfp4"
    res = pipeline.decode_step(case)
    for b in range(spec.B):
        e = int(case["pos"][b])
        k = f64(case["xi_new"][b])
        km = mx.dequantize(*mx.quantize(k))
        assert not np.array_equal(km, k)
        # on the grid: each block's values are multiples of 2^(s-1) of magnitude <= 6 * 2^s
        for blk in range(2):
            v = km[32 * blk:32 * blk + 32]
            s = mx.shared_exponent(k[32 * blk:32 * blk + 32])
            assert np.all(np.abs(v) <= 6 * 2.0 ** s)
            assert np.all(np.mod(v, 2.0 ** (s - 1)) == 0)
        s_mx, s_bf = res["scores"][b], bf["scores"][b]
        keep = np.arange(s_mx.size) != e
        np.testing.assert_array_equal(s_mx[keep], s_bf[keep])
        want = csa.index_scores(f64(case["q_idx"][b]), f64(case["w"][b]), km[None])[0]
        assert s_mx[e] == want


def test_gap_enforcement_decode():
    case = small_decode(case_id=905, L=8192, ragged=False)
    gaps.enforce_decode(case)
    res = pipeline.decode_step(case)
    for b, s in res["scores"].items():
        assert gaps.gap_ok(s, case["spec"].K)
    again = small_decode(case_id=905, L=8192, ragged=False)
    gaps.enforce_decode(again)
    assert torch.equal(case["w"], again["w"])        # redraws are deterministic


def test_gap_enforcement_hierarchical():
    case = small_decode(case_id=906, m=1, L=2000, block_size=4, max_blocks=64, ragged=False, K=32)
    gaps.enforce_decode(case)
    res = pipeline.decode_step(case)
    for b in res["scores"]:
        assert gaps.gap_ok(csa.block_maxima(res["scores"][b], 4), 64)
        assert gaps.gap_ok(res["scores2"][b], 32)


def test_gap_ok_rule():
    assert gaps.gap_ok(np.array([3.0, 2.0, 1.0]), 3)
    assert gaps.gap_ok(np.array([1.0, 0.998, 0.0]), 1)
    assert not gaps.gap_ok(np.array([1.0, 0.9995, 0.0]), 1)
    assert not gaps.gap_ok(np.array([0.0, 0.0, 5.0]), 2)     # exact tie at the boundary


def test_prefill_rows_and_gaps():
    spec = datagen.CaseSpec(907, "prefill", B=1, L=512, m=4, H_I=8, d_I=16, H=4, D=32, K=16,
                            W=8, w_cap=128, chunk=64)
    case = datagen.make_case(spec)
    rows = [(0, 0), (0, 17), (0, 63)]
    gaps.enforce_prefill(case, rows)
    res = pipeline.prefill_rows(case, rows)
    kv_c, ki_c = pipeline.prefill_entries(case)
    assert kv_c.shape == (1, 16, 32)
    for (b, i), ids in res["ids"].items():
        t = int(case["q_pos"][b, i])
        n = csa.n_visible(t, 4, spec.entries)
        assert ids[ids >= 0].max() < n and (ids >= 0).sum() == min(16, n)
        assert gaps.gap_ok(res["scores"][(b, i)], 16)


def test_tiny_forward_runs_and_gaps():
    spec = datagen.CaseSpec(908, "tiny", dtype="f32", B=1, L=256, m=4, H_I=4, d_I=32, H=4,
                            D=64, K=16, W=16, w_cap=256, unit_scale=False, bias_sigma=0.1,
                            scale=0.125)
    case = datagen.make_case(spec)
    gaps.enforce_tiny(case)
    res = pipeline.tiny_forward(case)
    for (b, i), s in res["scores"].items():
        assert gaps.gap_ok(s, 16)
    # query 0 sees no entry and only its own row: the output is the sink-weighted row 0
    x0 = f64(case["x"][0, 0])
    z = 0.125 * (f64(case["q"][0, 0]) @ x0)
    wgt = 1 / (1 + np.exp(f64(case["sink"]) - z))
    np.testing.assert_allclose(res["out"][(0, 0)], csa.round_f32(wgt[:, None] * x0), rtol=1e-6)


def test_bf16_scores_rank_rounded_values_ties_to_lower_id():
    # scores 1.0 + 2^-10 and 1.0 round to the same bf16 value 1.0 (spacing 2^-7): with BF16
    # scores the lower id wins the last place, with fp32 scores the larger score does
    s = np.array([0.5, 1.0, 3.0, 1.0 + 2.0 ** -10, 0.25])
    assert csa.select_topk(s, 2).tolist() == [2, 3]
    sb = csa.round_bf16(csa.round_f32(s))
    assert sb[1] == sb[3] == 1.0
    assert csa.select_topk(sb, 2).tolist() == [1, 2]


def test_gap_rule_bf16():
    # K = 2 over 4 scores; the 2nd bf16 value is 1.0; a score on the midpoint 1 + 2^-8 between
    # 1.0 and its upper neighbour 1 + 2^-7 is ambiguous, one 2^-12 away from it is not
    base = np.array([3.0, 1.0, 0.25, 0.125])
    assert gaps.gap_ok_bf16(base, 2)
    amb = base.copy(); amb[3] = 1.0 + 2.0 ** -8
    assert not gaps.gap_ok_bf16(amb, 2)
    ok = base.copy(); ok[3] = 1.0 + 2.0 ** -8 + 2.0 ** -12
    assert gaps.gap_ok_bf16(ok, 2)
    # below a power of two the spacing halves: the midpoint under 1.0 is 1 - 2^-9
    low = base.copy(); low[3] = 1.0 - 2.0 ** -9
    assert not gaps.gap_ok_bf16(low, 2)
    assert gaps.gap_ok_bf16(np.array([1.0, 2.0]), 2)       # no more scores than K


def test_decode_step_bf16_scores():
    case = small_decode(case_id=906, B=4, L=8192, d_I=64, H_I=8, K=64, ragged=False)
    spec = case["spec"]
    case["score_format"] = "bf16"
    gaps.enforce_decode(case)
    res = pipeline.decode_step(case)
    for b in range(spec.B):
        s = res["scores"][b]
        assert np.array_equal(s, csa.round_bf16(s))          # ranked on bf16 values
        ids = res["ids"][b]
        sel = np.zeros(s.size, bool); sel[ids] = True
        # every selected score reaches every unselected one, and at the K-th value the
        # selected ids are the lowest of that value
        assert s[sel].min() >= s[~sel].max()
        v = s[sel].min()
        tie_sel = np.flatnonzero(sel & (s == v)); tie_out = np.flatnonzero(~sel & (s == v))
        assert tie_out.size == 0 or tie_sel.max() < tie_out.min()
    # the same inputs ranked on fp32 scores keep most of the same entries
    f32b = pipeline.decode_step({**case, "score_format": "f32"})
    rec = np.mean([np.isin(res["ids"][b], f32b["ids"][b]).mean() for b in range(spec.B)])
    assert rec > 0.9


@pytest.mark.parametrize("fmt,enc", [("fp8", fp8), ("fp4", kv_fp4)])
def test_quantised_cache_attends_the_new_entry_at_its_cached_value(fmt, enc):
    # m = 1: the new entry is the raw row x_new (a softmax over one logit). With an FP8 (E4M3 /
    # bf16) or FP4 (E2M1 x E4M3 block scale) main cache the step must attend to it at its cached
    # value: the same outputs as the dtype path given that value as x_new, and not those of the
    # unquantised entry
    case = small_decode(case_id=906, m=1, L=12, D=512, H=2, ragged=False)   # K >= entries
    spec = case["spec"]
    case["kv"] = torch.from_numpy(enc.cached_entries(f64(case["kv"]))).to(case["kv"].dtype)
    plain = pipeline.decode_step(case)
    case8 = dict(case, kv_format=fmt)
    res = pipeline.decode_step(case8)
    xq = enc.cached_entries(f64(case["x_new"]))
    assert not np.array_equal(xq, f64(case["x_new"]))
    moved = dict(case, x_new=torch.from_numpy(xq).to(case["x_new"].dtype))
    want = pipeline.decode_step(moved)
    differs = False
    for b in range(spec.B):
        np.testing.assert_array_equal(res["kv_new"][b], plain["kv_new"][b])
        np.testing.assert_array_equal(res["ids"][b], plain["ids"][b])
        for c in range(spec.n_attn):
            np.testing.assert_array_equal(res["out"][b][c], want["out"][b][c])
            differs |= not np.array_equal(res["out"][b][c], plain["out"][b][c])
    assert differs


def test_new_entry_norm_and_rope():
    # RMSNorm with a unit gamma gives the stored entry a unit mean square (up to its bf16
    # rounding); RoPE alone keeps the first channels and the entry's L2 norm, and turns the
    # last 64 pairwise; every other entry and the ids' inputs are unchanged
    case = small_decode(case_id=907, m=1, L=40, D=512, H=2, ragged=False)
    spec = case["spec"]
    plain = pipeline.decode_step(case)
    normed = pipeline.decode_step(dict(case, kv_gamma=torch.ones(512, dtype=case["kv"].dtype)))
    roped = pipeline.decode_step(dict(case, kv_rope_dim=64))
    for b in range(spec.B):
        e = normed["kv_new"][b]
        assert abs(np.mean(e ** 2) - 1.0) < 1e-2
        assert not np.allclose(e, plain["kv_new"][b])
        r, p = roped["kv_new_exact"][b], plain["kv_new"][b]
        np.testing.assert_array_equal(r[:448], p[:448])
        assert not np.allclose(r[448:], p[448:])
        np.testing.assert_allclose(np.hypot(r[448::2], r[449::2]),
                                   np.hypot(p[448::2], p[449::2]), rtol=1e-12)
        np.testing.assert_array_equal(roped["ids"][b], plain["ids"][b])
