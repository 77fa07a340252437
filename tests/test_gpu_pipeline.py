"""GPU parity of whole paths: the tiny fp32 forward (all 2,048 queries) and the fused decode
step (flat and hierarchical, several attention calls), against the float64 oracle."""
import numpy as np
import pytest
import torch

import datagen
import sparse_long_context_csa_amd as csa
from gpu_helpers import (assert_ids, assert_rows_close, check_step, dev, fp8_case, mxfp4_case,
                         quant_case, run_step)
from oracle import csa as ocsa
from oracle import gaps, pipeline
from oracle.pipeline import f64

pytestmark = pytest.mark.gpu


def test_tiny_forward_fp32():
    """The tiny workload: compress 2,048 raw rows 4:1, index with 4x32 heads, Top-64 under
    the causal limit, attend (window 64, sink) for every one of the 2,048 queries."""
    case = datagen.make_case(datagen.CONFIGS[1])
    gaps.enforce_tiny(case)
    spec = case["spec"]
    ref = pipeline.tiny_forward(case)
    kv = csa.compress(dev(case["x"]), dev(case["z"]), dev(case["bias"]), spec.m)
    idx = csa.index_topk(dev(case["q_idx"]), dev(case["w"]), dev(case["k_idx"]),
                         dev(case["q_pos"]), spec.m, spec.K, e_count=dev(case["e_count"]))
    out = csa.sparse_attn(dev(case["q"]), kv, idx, dev(case["x"]), spec.L, spec.W,
                          dev(case["q_pos"]), dev(case["sink"]), spec.softmax_scale)
    torch.cuda.synchronize()
    np.testing.assert_allclose(f64(kv.cpu()), ref["kv"], rtol=2e-6, atol=1e-6)
    idx, out = idx.cpu(), out.cpu()
    for (b, i), ids in ref["ids"].items():
        assert_ids(idx[b, i].numpy(), ids, f"query {i}")
        assert_rows_close(f64(out[b, i]), ref["out"][(b, i)], 2e-2, f"query {i}")


def test_decode_step_flat_ragged():
    spec = datagen.CaseSpec(7100, "decode", B=5, L=24000, m=4, w_cap=256, ragged=True)
    case = datagen.make_case(spec)
    gaps.enforce_decode(case)
    ref = pipeline.decode_step(case)
    step, st, rings, out, idx = run_step(case)
    check_step(case, ref, st, rings, out, idx)
    # the same step again (idempotent state) is bitwise identical
    out2, idx2 = step()
    torch.cuda.synchronize()
    assert torch.equal(idx2.cpu(), idx)
    assert torch.equal(out2[0].cpu(), out[0])


def test_decode_step_hierarchical_three_calls():
    spec = datagen.CaseSpec(7101, "decode", B=3, L=40000, m=1, w_cap=128, block_size=8,
                            max_blocks=512, n_attn=3, ragged=True)
    case = datagen.make_case(spec)
    gaps.enforce_decode(case)
    ref = pipeline.decode_step(case)
    _, st, rings, out, idx = run_step(case)
    check_step(case, ref, st, rings, out, idx)


def test_decode_step_incomplete_block_writes_no_entry():
    spec = datagen.CaseSpec(7102, "decode", B=4, L=9000, m=4, w_cap=128, ragged=True)
    case = datagen.make_case(spec)
    gaps.enforce_decode(case)
    ref = pipeline.decode_step(case)
    kv0 = case["kv"].clone()
    _, st, rings, out, idx = run_step(case)
    check_step(case, ref, st, rings, out, idx)
    for b in range(spec.B):
        t = int(case["pos"][b])
        if (t + 1) % 4:
            assert torch.equal(st["kv"][b].cpu(), kv0[b])


# Flat steps over caches of more than 32,768 entries: the scan leaves per-chunk candidate
# segments and the select works on them.
def test_decode_step_segments_ragged():
    spec = datagen.CaseSpec(7110, "decode", B=3, L=4 * 60000, m=4, w_cap=256, ragged=True)
    case = datagen.make_case(spec)
    gaps.enforce_decode(case)
    ref = pipeline.decode_step(case)
    _, st, rings, out, idx = run_step(case)
    check_step(case, ref, st, rings, out, idx)


def test_decode_step_segments_short_rows():
    # a cache of 40,000 entries holding 300 to 600 visible ones: some rows see fewer than
    # K = 512 (all selected, -1 padded), the others take the segments of a few chunks
    spec = datagen.CaseSpec(7111, "decode", B=4, L=2400, e_cap=40000, m=4, w_cap=128,
                            ragged=True)
    case = datagen.make_case(spec)
    gaps.enforce_decode(case)
    ref = pipeline.decode_step(case)
    assert any(int(ref["ids"][b][-1]) == -1 for b in range(spec.B))
    _, st, rings, out, idx = run_step(case)
    check_step(case, ref, st, rings, out, idx)


def test_decode_step_segments_clustered_winners():
    # a doubled stretch of indexer keys (exactly doubled scores) concentrates the Top-K in a
    # few chunks whose own thresholds exceed the K-th key: the streaming select takes over
    spec = datagen.CaseSpec(7112, "decode", B=2, L=4 * 50000, m=4, w_cap=128)
    case = datagen.make_case(spec)
    k = case["k_idx"]
    k[0, 20000:21500] = (k[0, 20000:21500].float() * 2).to(k.dtype)
    k[1, 7000:7300] = (k[1, 7000:7300].float() * 2).to(k.dtype)
    gaps.enforce_decode(case)
    ref = pipeline.decode_step(case)
    ids0 = ref["ids"][0]
    assert np.sum((ids0 >= 20000) & (ids0 < 21500)) > 200
    _, st, rings, out, idx = run_step(case)
    check_step(case, ref, st, rings, out, idx)


def test_decode_step_segments_odd_k_and_window():
    # K = 500 and W = 100: one tile holds the last selected ids and the first window rows
    spec = datagen.CaseSpec(7113, "decode", B=2, L=4 * 40000, m=4, K=500, W=100, w_cap=128,
                            ragged=True)
    case = datagen.make_case(spec)
    gaps.enforce_decode(case)
    ref = pipeline.decode_step(case)
    _, st, rings, out, idx = run_step(case)
    check_step(case, ref, st, rings, out, idx)


# MXFP4 indexer cache: the scan dequantises 64-key tiles of codes and scale bytes (or, with the
# query in FP4 too, multiplies the codes by the FP4 query in the scaled MFMA); the entry a step
# completes is pooled, quantised and stored by the scan.
@pytest.mark.parametrize("query", ["bf16", "fp4"])
@pytest.mark.parametrize("spec", [
    datagen.CaseSpec(7120, "decode", B=5, L=24000, m=4, w_cap=256, ragged=True),
    datagen.CaseSpec(7121, "decode", B=3, L=4 * 60000, m=4, w_cap=256, ragged=True),
    datagen.CaseSpec(7122, "decode", B=4, L=2400, e_cap=40000, m=4, w_cap=128, ragged=True),
    datagen.CaseSpec(7123, "decode", B=3, L=20000, m=1, w_cap=128, ragged=True),
], ids=["flat", "segments", "short_rows", "m1"])
def test_decode_step_mxfp4_keys(spec, query):
    case, idx_state = mxfp4_case(spec)
    if query == "fp4":
        case["idx_format"] = "mxfp4_qk"
    gaps.enforce_decode(case)
    ref = pipeline.decode_step(case)
    step, st, rings, out, idx = run_step(case, idx_state)
    check_step(case, ref, st, rings, out, idx)
    # entries the step did not complete are untouched
    for b in range(spec.B):
        t = int(case["pos"][b])
        keep = np.ones(st["k_idx"].shape[1], bool)
        if (t + 1) % spec.m == 0:
            keep[(t + 1) // spec.m - 1] = False
        assert torch.equal(st["k_idx"][b].cpu()[keep], idx_state["k_idx"][b].cpu()[keep])
        assert torch.equal(st["k_idx_scale"][b].cpu()[keep],
                           idx_state["k_idx_scale"][b].cpu()[keep])
    out2, idx2 = step()
    torch.cuda.synchronize()
    assert torch.equal(idx2.cpu(), idx)


@pytest.mark.parametrize("spec", [
    # a cache capacity that is not a multiple of the 64-key tile, rows ragged below it
    datagen.CaseSpec(7124, "decode", B=3, L=4 * 40003, e_cap=40003, m=4, w_cap=128,
                     ragged=True),
    datagen.CaseSpec(7125, "decode", B=2, L=8 * 5000, m=8, w_cap=128, ragged=True),
    datagen.CaseSpec(7126, "decode", B=2, L=2 * 30000, m=2, K=500, W=100, w_cap=128,
                     ragged=True),
], ids=["e_cap_40003", "m8", "m2_odd_k"])
@pytest.mark.parametrize("query", ["bf16", "fp4"])
def test_decode_step_mxfp4_keys_edges(spec, query):
    case, idx_state = mxfp4_case(spec)
    if query == "fp4":
        case["idx_format"] = "mxfp4_qk"
    gaps.enforce_decode(case)
    ref = pipeline.decode_step(case)
    _, st, rings, out, idx = run_step(case, idx_state)
    check_step(case, ref, st, rings, out, idx)


@pytest.mark.parametrize("fmt", ["mxfp4_keys", "bf16_scores"])
def test_decode_step_clustered_winners_formats(fmt):
    # the Top-K concentrated in a few chunks (their thresholds exceed the K-th key): the select
    # streams over the full scores, with MXFP4 keys or with bf16 scores
    spec = datagen.CaseSpec(7112, "decode", B=2, L=4 * 50000, m=4, w_cap=128)
    case = datagen.make_case(spec)
    k = case["k_idx"]
    k[0, 20000:21500] = (k[0, 20000:21500].float() * 2).to(k.dtype)
    k[1, 7000:7300] = (k[1, 7000:7300].float() * 2).to(k.dtype)
    idx_state = None
    if fmt == "mxfp4_keys":
        from oracle import mx
        codes, scales = mx.quantize(f64(k))
        kq = torch.from_numpy(mx.dequantize(codes, scales)).to(k.dtype)
        kc, ks = csa.quantize_mxfp4(dev(k))
        case["k_idx"] = kq
        case["idx_format"] = "mxfp4"
        idx_state = {"k_idx": kc, "k_idx_scale": ks}
    else:
        case["score_format"] = "bf16"
    gaps.enforce_decode(case)
    ref = pipeline.decode_step(case)
    ids0 = ref["ids"][0]
    assert np.sum((ids0 >= 20000) & (ids0 < 21500)) > 100   # far above 512 / 25 chunks
    _, st, rings, out, idx = run_step(case, idx_state)
    check_step(case, ref, st, rings, out, idx)


# BF16 index scores: the scan rounds every score to bf16 before it leaves; the selection (ties
# at the K-th value to the lower id) must match the oracle's ranking of its fp32 scores rounded
# to bf16, id for id.
@pytest.mark.parametrize("keys", ["bf16", "mxfp4", "mxfp4_qk"])
@pytest.mark.parametrize("spec", [
    datagen.CaseSpec(7130, "decode", B=5, L=24000, m=4, w_cap=256, ragged=True),
    datagen.CaseSpec(7131, "decode", B=3, L=4 * 60000, m=4, w_cap=256, ragged=True),
    datagen.CaseSpec(7132, "decode", B=4, L=2400, e_cap=40000, m=4, w_cap=128, ragged=True),
], ids=["flat", "segments", "short_rows"])
def test_decode_step_bf16_scores(spec, keys):
    if keys.startswith("mxfp4"):
        case, idx_state = mxfp4_case(spec)
        case["idx_format"] = keys
    else:
        case, idx_state = datagen.make_case(spec), None
    case["score_format"] = "bf16"
    gaps.enforce_decode(case)
    ref = pipeline.decode_step(case)
    _, st, rings, out, idx = run_step(case, idx_state)
    check_step(case, ref, st, rings, out, idx)


@pytest.mark.parametrize("spec", [
    datagen.CaseSpec(7140, "decode", B=5, L=24000, m=4, w_cap=256, ragged=True),      # splits
    datagen.CaseSpec(7141, "decode", B=3, L=40000, m=1, w_cap=128, block_size=8,
                     max_blocks=512, n_attn=3, ragged=True),
    # 260 rows: one workgroup per row, the output leaves from the attention kernel itself
    datagen.CaseSpec(7142, "decode", B=260, L=3000, m=4, w_cap=128, ragged=True),
    datagen.CaseSpec(7143, "decode", dtype="f32", B=2, L=5000, m=4, w_cap=128, ragged=True),
], ids=["flat", "hier_three_calls", "rows_260", "f32_generic"])
def test_decode_step_output_rope(spec):
    """The queries' RMSNorm and RoPE (at +t), prepared by the selection launch's side
    workgroups, and the inverse RoPE (at -t, last 64 channels of each head) fused into the
    attention's output store: outputs against the oracle's."""
    case = datagen.make_case(spec)
    case["out_rope_dim"] = 64
    case["q_rope_dim"] = 64
    case["q_gamma"] = [datagen.tensor(spec.case_id, 90 + c, (spec.D,), spec.dtype, 0.3) + 1.0
                       for c in range(spec.n_attn)]
    case["q_gamma"][0] = case["q_gamma"][0].to(case["q"][0].dtype)
    gaps.enforce_decode(case)
    ref = pipeline.decode_step(case)
    _, st, rings, out, idx = run_step(case)
    check_step(case, ref, st, rings, out, idx)


@pytest.mark.parametrize("fused", [True, False], ids=["side_workgroups", "separate_ingest"])
def test_decode_step_query_norm_some_calls(fused):
    """RMSNorm on the queries of calls 0 and 2 only, no query RoPE: call 1 attends with its own
    query unchanged. bf16 64 x 128 runs the prep in the selection launch; the fp32 case (no
    fused ingest) runs it as separate passes."""
    spec = (datagen.CaseSpec(7144, "decode", B=3, L=30000, m=4, w_cap=128, block_size=8,
                             max_blocks=512, n_attn=3, ragged=True) if fused else
            datagen.CaseSpec(7145, "decode", dtype="f32", B=2, L=6000, m=4, w_cap=128,
                             n_attn=3, ragged=True))
    case = datagen.make_case(spec)
    g = [datagen.tensor(spec.case_id, 90 + c, (spec.D,), spec.dtype, 0.3) + 1.0
         for c in range(spec.n_attn)]
    case["q_gamma"] = [g[0].to(case["q"][0].dtype), None, g[2].to(case["q"][0].dtype)]
    gaps.enforce_decode(case)
    ref = pipeline.decode_step(case)
    _, st, rings, out, idx = run_step(case)
    check_step(case, ref, st, rings, out, idx)


def test_decode_step_scan_events():
    """The scan kernel's dispatch takes the step's scan events: the result is unchanged and
    their interval lies inside the step's own (marker events 0 and 4)."""
    spec = datagen.CaseSpec(7114, "decode", B=2, L=4 * 40000, m=4, w_cap=128)
    case = datagen.make_case(spec)
    gaps.enforce_decode(case)
    ref = pipeline.decode_step(case)
    step, st, rings, out, idx = run_step(case)
    check_step(case, ref, st, rings, out, idx)
    ev = csa.HipEvents()
    marks = [ev.create() for _ in range(5)]
    s0, s1 = ev.create(), ev.create()
    try:
        step.set_events(marks)
        step.set_scan_events(s0, s1)
        out2, idx2 = step()
        torch.cuda.synchronize()
        assert torch.equal(idx2.cpu(), idx)
        scan = ev.ms(s0, s1)
        whole = ev.ms(marks[0], marks[4])
        assert 0.0 < scan < whole
        with pytest.raises(ValueError):
            step.set_scan_events(s0, None)
    finally:
        step.set_events([])
        step.set_scan_events()
        for e in marks + [s0, s1]:
            ev.destroy(e)


@pytest.mark.parametrize("variant", ["flat", "hier", "segments"])
def test_decode_step_graph_replay_matches_eager(variant):
    """The fused step captured in a HIP graph: every replay (with eager work and
    synchronisations in between) reproduces the eager result bit for bit."""
    if variant == "hier":
        spec = datagen.CaseSpec(7103, "decode", B=2, L=20000, m=1, w_cap=128, block_size=8,
                                max_blocks=256, n_attn=2, ragged=True)
    elif variant == "flat":
        spec = datagen.CaseSpec(7104, "decode", B=3, L=40000, m=4, w_cap=128, ragged=True)
    else:
        spec = datagen.CaseSpec(7105, "decode", B=2, L=4 * 45000, m=4, w_cap=128, ragged=True)
    case = datagen.make_case(spec)
    gaps.enforce_decode(case)
    step, st, rings, out, idx = run_step(case)
    ref = pipeline.decode_step(case)
    check_step(case, ref, st, rings, out, idx)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        for o in step.out:
            o.zero_()
        step.out_idx.fill_(-7)
        junk.mul_(1.0001)                      # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out_idx.cpu(), idx), f"replay {rep}: ids differ"
        for c in range(spec.n_attn):
            assert torch.equal(step.out[c].cpu(), out[c]), f"replay {rep}: output {c} differs"


# FP8 / FP4 main cache: 576- or 288-byte entries; the attention expands them to bf16 on their
# way to the MFMA operands, the step stores the entry it completes in the cache's format.
@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
@pytest.mark.parametrize("spec,mx", [
    (datagen.CaseSpec(7150, "decode", B=5, L=24000, m=4, w_cap=256, ragged=True), False),
    (datagen.CaseSpec(7151, "decode", B=3, L=40000, m=1, w_cap=128, block_size=8,
                      max_blocks=512, n_attn=3, ragged=True), False),
    (datagen.CaseSpec(7152, "decode", B=260, L=3000, m=4, w_cap=128, ragged=True), False),
    (datagen.CaseSpec(7153, "decode", B=4, L=4 * 50000, m=4, w_cap=128, ragged=True), True),
], ids=["flat", "hier_three_calls", "rows_260", "with_mxfp4_keys"])
def test_decode_step_quantised_cache(spec, mx, fmt):
    if mx:
        case, state = mxfp4_case(spec)
    else:
        case, state = datagen.make_case(spec), {}
    state.update(quant_case(case, fmt))
    gaps.enforce_decode(case)
    ref = pipeline.decode_step(case)
    step, st, rings, out, idx = run_step(case, state)
    check_step(case, ref, st, rings, out, idx)
    # entries the step did not complete are untouched
    for b in range(spec.B):
        t = int(case["pos"][b])
        keep = np.ones(st["kv"].shape[1], bool)
        if (t + 1) % spec.m == 0:
            keep[(t + 1) // spec.m - 1] = False
        assert torch.equal(st["kv"][b].cpu()[keep], state["kv"][b].cpu()[keep])


# The entry a step completes gets its RMSNorm and RoPE at t before it is stored (and attended).
@pytest.mark.parametrize("spec,fp8", [
    (datagen.CaseSpec(7160, "decode", B=5, L=24000, m=4, w_cap=256, ragged=True), False),
    (datagen.CaseSpec(7161, "decode", B=3, L=40000, m=1, w_cap=128, block_size=8,
                      max_blocks=512, n_attn=3, ragged=True), False),
    (datagen.CaseSpec(7162, "decode", dtype="f32", B=2, L=6000, m=4, w_cap=128, ragged=True),
     False),
    (datagen.CaseSpec(7163, "decode", B=4, L=4 * 30000, m=4, w_cap=128, ragged=True), "fp8"),
    (datagen.CaseSpec(7164, "decode", B=4, L=4 * 30000, m=4, w_cap=128, ragged=True), "fp4"),
], ids=["flat", "hier_three_calls", "f32_separate_ingest", "fp8_cache", "fp4_cache"])
def test_decode_step_entry_norm_rope(spec, fp8):
    case = datagen.make_case(spec)
    state = quant_case(case, fp8) if fp8 else {}
    case["kv_gamma"] = (datagen.tensor(spec.case_id, 95, (spec.D,), spec.dtype, 0.3) + 1.0).to(
        case["x_new"].dtype)
    case["kv_rope_dim"] = 64
    # the completing sequences: the entry is attended in the step only when it is selected
    gaps.enforce_decode(case)
    ref = pipeline.decode_step(case)
    assert ref["kv_new"], "no sequence completes a block"
    _, st, rings, out, idx = run_step(case, state or None)
    check_step(case, ref, st, rings, out, idx)


# The overlapped two-stream main compressor inside the step: the b stream's new row enters its
# two-block ring, the entry a step completes pools its block's a rows with the previous block's
# b rows (none for a sequence's first entry); the indexer keys keep the single stream.
@pytest.mark.parametrize("spec,fmt", [
    (datagen.CaseSpec(7170, "decode", B=5, L=24000, m=4, w_cap=256, ragged=True,
                      compressor="c4a"), None),
    (datagen.CaseSpec(7171, "decode", B=4, L=2000, m=4, w_cap=128, compressor="c4a"), None),
    (datagen.CaseSpec(7172, "decode", B=2, L=4, e_cap=4096, m=4, w_cap=128,
                      compressor="c4a"), None),
    (datagen.CaseSpec(7173, "decode", B=3, L=40000, m=1, w_cap=128, block_size=8,
                      max_blocks=512, n_attn=3, ragged=True, compressor="c4a"), None),
    (datagen.CaseSpec(7174, "decode", B=4, L=4 * 50000, m=4, w_cap=128, ragged=True,
                      compressor="c4a"), "mxfp4"),
    (datagen.CaseSpec(7175, "decode", dtype="f32", B=3, L=6000, m=4, w_cap=128, ragged=True,
                      compressor="c4a"), None),
    (datagen.CaseSpec(7176, "decode", B=4, L=2 * 30000, m=2, w_cap=128, ragged=True,
                      compressor="c4a"), "fp8_prep"),
    (datagen.CaseSpec(7177, "decode", B=3, L=8 * 3000, m=8, w_cap=128, ragged=True,
                      compressor="c4a"), None),
    (datagen.CaseSpec(7178, "decode", B=4, L=4 * 30000, m=4, w_cap=128, ragged=True,
                      compressor="c4a"), "fp4_prep"),
], ids=["flat", "all_selected", "first_entry", "hier_three_calls", "mxfp4_keys",
        "f32_separate_ingest", "fp8_cache_norm_rope", "m8_two_pass", "fp4_cache_norm_rope"])
def test_decode_step_overlapped_compressor(spec, fmt):
    if fmt == "mxfp4":
        case, state = mxfp4_case(spec)
    else:
        case, state = datagen.make_case(spec), {}
    if fmt in ("fp8_prep", "fp4_prep"):
        state.update(quant_case(case, fmt[:3]))
        case["kv_gamma"] = (datagen.tensor(spec.case_id, 95, (spec.D,), spec.dtype, 0.3)
                            + 1.0).to(case["x_new"].dtype)
        case["kv_rope_dim"] = 64
    gaps.enforce_decode(case)
    ref = pipeline.decode_step(case)
    assert ref["kv_new"], "no sequence completes a block"
    step, st, rings, out, idx = run_step(case, state or None)
    check_step(case, ref, st, rings, out, idx)
    if spec.L == 2000:   # every entry selected: the new entry takes part in the attention
        for b in range(spec.B):
            assert (spec.L // spec.m - 1) in idx[b].tolist()
