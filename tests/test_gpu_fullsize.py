"""GPU parity at the full sizes of the five workloads, in the launch configuration the bench
times: every sequence of the decode workloads, and 376 sampled query rows of the chunked
prefill (the oracle computes those one by one)."""
import dataclasses

import numpy as np
import pytest
import torch

import datagen
import sparse_long_context_csa_amd as csa
from gpu_helpers import (assert_ids, assert_pooled, assert_rows_close, assert_scores, check_step,
                         dev, fp8_case, mxfp4_case, pooled_xmax, quant_case, run_step)
from oracle import csa as ocsa
from oracle import gaps, pipeline
from oracle.pipeline import f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [2, 4, 5])
def test_decode_workload_fullsize(cfg):
    case = datagen.make_case(datagen.CONFIGS[cfg])
    print(f"config {cfg}: inputs ready", flush=True)
    gaps.enforce_decode(case)
    _, st, rings, out, idx = run_step(case)
    ref = pipeline.decode_step(case)
    check_step(case, ref, st, rings, out, idx)


def test_decode_1m_overlapped_compressor():
    """The 1M-context decode workload with the overlapped two-stream main compressor (the
    bench's --compressor c4a line)."""
    case = datagen.make_case(dataclasses.replace(datagen.CONFIGS[4], compressor="c4a"))
    print("config 4 (c4a): inputs ready", flush=True)
    gaps.enforce_decode(case)
    _, st, rings, out, idx = run_step(case)
    ref = pipeline.decode_step(case)
    check_step(case, ref, st, rings, out, idx)


@pytest.mark.parametrize("query", ["bf16", "fp4"])
@pytest.mark.parametrize("cfg", [2, 4])
def test_decode_workload_fullsize_mxfp4_keys(cfg, query):
    """The flat decode workloads with the indexer cache in MXFP4 (the bench's --idx-format
    mxfp4 line) and, with query "fp4", the indexer query in MXFP4 too (--idx-format
    mxfp4qk): the GPU quantises the generated keys, the oracle scores their MXFP4 values."""
    case, idx_state = mxfp4_case(datagen.CONFIGS[cfg])
    if query == "fp4":
        case["idx_format"] = "mxfp4_qk"
    print(f"config {cfg} (MXFP4 keys): inputs ready", flush=True)
    gaps.enforce_decode(case)
    _, st, rings, out, idx = run_step(case, idx_state)
    ref = pipeline.decode_step(case)
    check_step(case, ref, st, rings, out, idx)


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_decode_1m_quantised_main_cache(fmt):
    """The 1M-context decode workload over an FP8 or FP4 main cache (the bench's --kv-format
    lines): the GPU quantises the generated entries, the oracle attends their cached values."""
    case = datagen.make_case(datagen.CONFIGS[4])
    state = quant_case(case, fmt)
    print(f"config 4 ({fmt} main cache): inputs ready", flush=True)
    gaps.enforce_decode(case)
    _, st, rings, out, idx = run_step(case, state)
    ref = pipeline.decode_step(case)
    check_step(case, ref, st, rings, out, idx)


@pytest.mark.parametrize("compressor", ["single", "c4a"])
def test_decode_workload_fullsize_every_format_and_fusion(compressor):
    """The 8 x 65,536-token decode workload with every production format and fusion at once:
    FP8 main cache, MXFP4 indexer keys, BF16 index scores, the queries' and the completed
    entry's RMSNorm + RoPE and the inverse RoPE on the output (the GPU quantises the caches;
    the oracle holds their FP8 / MXFP4 values from its own encoders); with either main
    compressor."""
    spec = dataclasses.replace(datagen.CONFIGS[2], compressor=compressor)
    case, state = mxfp4_case(spec)
    state.update(fp8_case(case))
    case["score_format"] = "bf16"
    case["q_rope_dim"] = case["out_rope_dim"] = case["kv_rope_dim"] = 64
    case["q_gamma"] = [(datagen.tensor(spec.case_id, 90, (spec.D,), spec.dtype, 0.3) + 1.0).to(
        case["x_new"].dtype)]
    case["kv_gamma"] = (datagen.tensor(spec.case_id, 95, (spec.D,), spec.dtype, 0.3) + 1.0).to(
        case["x_new"].dtype)
    print("config 2 (all formats and fusions): inputs ready", flush=True)
    gaps.enforce_decode(case)
    _, st, rings, out, idx = run_step(case, state)
    ref = pipeline.decode_step(case)
    check_step(case, ref, st, rings, out, idx)


PREFILL_ROWS = sorted(set(range(64)) | set(range(4032, 4096)) | set(range(0, 4096, 16)))


def _prefill_run(case, g, kv, ki):
    spec = case["spec"]
    idx, scores = csa.index_topk(g["q_idx"], g["w"], ki, g["q_pos"], spec.m, spec.K,
                                 e_count=g["e_count"], want_all=True)
    out = csa.sparse_attn(g["q"], kv, idx, g["ring"], spec.w_cap, spec.W, g["q_pos"], g["sink"],
                          spec.softmax_scale)
    torch.cuda.synchronize()
    return idx.cpu(), scores, out.float().cpu()


def _prefill_check(case, rows, kv_c, ki_c, idx, scores, out, what):
    spec = case["spec"]
    e0 = (spec.L - spec.chunk) // spec.m
    ref = pipeline.prefill_rows(case, rows, kv_c, ki_c)
    ki = f64(case["k_idx"][0]).copy()
    ki[e0:e0 + ki_c.shape[1]] = f64(ki_c[0])
    for (b, i), ids in ref["ids"].items():
        assert_ids(idx[b, i].numpy(), ids, f"{what}: query row {i}")
        n = ocsa.n_visible(int(case["q_pos"][b, i]), spec.m, spec.entries)
        sg = f64(scores[b, i, :n].cpu())
        assert_scores(sg, ref["scores"][(b, i)],
                      ocsa.score_scale(f64(case["q_idx"][b, i]), f64(case["w"][b, i]), ki[:n]),
                      1e-3, f"{what}: scores of query row {i}")
        assert_rows_close(f64(out[b, i]), ref["out"][(b, i)], 2e-2, f"{what}: query row {i}")


def test_prefill_workload_fullsize():
    """Compress the 4,096-token chunk into both caches (checked against the exact pooled
    values), then index, select and attend all 4,096 queries. Checked on 256 query rows (every
    row of the first and last 64-query groups, every 16th row): ids, every index score of the
    row and the outputs. Pass 1 indexes over caches that hold the oracle's stored chunk
    entries (an ulp of pooling rounding cannot move a selection); pass 2 over the GPU's own
    pooled entries, with the gap rule enforced on the keys that pass uses."""
    spec = datagen.CONFIGS[3]
    case = datagen.make_case(spec)
    rows = [(0, i) for i in PREFILL_ROWS]
    assert len(rows) >= 256
    gaps.enforce_prefill(case, rows)
    print("config 3: inputs ready", flush=True)
    g = {k: dev(v) for k, v in case.items() if isinstance(v, torch.Tensor)}
    e0 = (spec.L - spec.chunk) // spec.m
    ne = spec.chunk // spec.m
    kv, ki = g["kv"].clone(), g["k_idx"].clone()
    csa.compress(g["x_chunk"], g["z_chunk"], g["bias"], spec.m, out=kv[:, e0:e0 + ne],
                 out_seq_stride=spec.entries * spec.D)
    csa.compress(g["xi_chunk"], g["zi_chunk"], g["bias_i"], spec.m, out=ki[:, e0:e0 + ne],
                 out_seq_stride=spec.entries * spec.d_I)
    torch.cuda.synchronize()
    for cache, xs, zs, bs in ((kv, "x_chunk", "z_chunk", "bias"),
                              (ki, "xi_chunk", "zi_chunk", "bias_i")):
        exact = ocsa.compress(f64(case[xs]), f64(case[zs]), f64(case[bs]), spec.m)
        assert_pooled(f64(cache[:, e0:e0 + ne].float().cpu()), exact,
                      pooled_xmax(f64(case[xs]), spec.m), f"chunk entries ({xs})")
    kv_gpu, ki_gpu = kv[:, e0:e0 + ne].cpu(), ki[:, e0:e0 + ne].cpu()
    # pass 1: the oracle's stored chunk entries in both caches
    kv_c, ki_c = pipeline.prefill_entries(case)
    kv1, ki1 = kv.clone(), ki.clone()
    kv1[:, e0:e0 + ne] = torch.from_numpy(kv_c).to(kv.dtype).to(kv.device)
    ki1[:, e0:e0 + ne] = torch.from_numpy(ki_c).to(ki.dtype).to(ki.device)
    idx, scores, out = _prefill_run(case, g, kv1, ki1)
    print("config 3 pass 1: GPU done", flush=True)
    _prefill_check(case, rows, kv_c, ki_c, idx, scores, out, "oracle chunk entries")
    del scores
    # pass 2: the GPU's own pooled chunk entries feed the index; the gates of a quarter of the
    # rows are fixed again for these keys
    rows2 = [(0, i) for i in PREFILL_ROWS[::4]]
    gaps.enforce_prefill(case, rows2, ki_c=ki_gpu)
    g["w"] = dev(case["w"])
    idx, scores, out = _prefill_run(case, g, kv, ki)
    print("config 3 pass 2: GPU done", flush=True)
    _prefill_check(case, rows2, f64(kv_gpu), f64(ki_gpu), idx, scores, out,
                   "GPU-pooled chunk entries")


def test_decode_1m_ragged_rows():
    """The 1M-context decode shape (262,144-entry caches, log-normal key norms) with ragged
    positions over [L/2, L): rows whose later scan items lie wholly or partly past the visible
    count, so the scan skips their tile loads; ids, outputs and state against the oracle."""
    spec = dataclasses.replace(datagen.CONFIGS[4], case_id=7400, ragged=True)
    case = datagen.make_case(spec)
    pos = case["pos"].tolist()
    assert min(pos) < spec.L - spec.L // 4 and max(pos) == spec.L - 1
    print(f"ragged 1M decode: positions {pos}", flush=True)
    gaps.enforce_decode(case)
    _, st, rings, out, idx = run_step(case)
    ref = pipeline.decode_step(case)
    check_step(case, ref, st, rings, out, idx)


def test_hca_decode_fullsize():
    """Heavily Compressed Attention at 1M context (m' = 128, 8,192 entries per sequence): the
    completed 128-row block is pooled by csa_compress into the cache, then csa_sparse_attn
    attends to every visible entry (top_k = all 8,192) plus the window and the sink. The oracle's
    decode step with K >= the visible count selects every entry, which is the dense form."""
    spec = datagen.HCA_DECODE
    case = datagen.make_case(spec)
    print("HCA: inputs ready", flush=True)
    ref = pipeline.decode_step(case)
    g = {k: dev(v) for k, v in case.items() if isinstance(v, torch.Tensor)}
    B, m, E, D = spec.B, spec.m, spec.entries, spec.D
    pos = case["pos"]
    kv = g["kv"].clone()
    ring = dev(case["rings"][0]).clone()
    xb, zb = g["x_tail"].clone(), g["z_tail"].clone()
    n_vis = []
    for b in range(B):
        t = int(pos[b])
        xb[b, t % m] = g["x_new"][b]
        zb[b, t % m] = g["z_new"][b]
        ring[b, t % spec.w_cap] = g["x_new"][b]
        n_vis.append(ocsa.n_visible(t, m, E))
    e_new = [(int(pos[b]) + 1) // m - 1 for b in range(B)]
    assert len(set(e_new)) == 1 and all((int(pos[b]) + 1) % m == 0 for b in range(B))
    csa.compress(xb, zb, g["bias"], m, out=kv[:, e_new[0]:], out_seq_stride=E * D)
    idx = torch.full((B, 1, E), -1, dtype=torch.int32)
    for b in range(B):
        idx[b, 0, :n_vis[b]] = torch.arange(n_vis[b], dtype=torch.int32)
    out = csa.sparse_attn(dev(case["q"][0]).unsqueeze(1), kv, dev(idx), ring, spec.w_cap,
                          spec.W, g["pos"].view(B, 1), dev(case["sink"][0]), case["scale"])
    torch.cuda.synchronize()
    for b in range(B):
        assert ref["ids"][b].tolist() == list(range(n_vis[b])) + [-1] * (E - n_vis[b])
        x = f64(case["x_tail"][b]).copy()
        x[int(pos[b]) % m] = f64(case["x_new"][b])
        assert_pooled(f64(kv[b, e_new[b]].cpu()), ocsa.compress(
            x, np.where(np.arange(m)[:, None] == int(pos[b]) % m, f64(case["z_new"][b]),
                        f64(case["z_tail"][b])), f64(case["bias"]), m)[0],
            np.abs(x).max(axis=0), f"HCA entry of seq {b}", m=m)
        assert_rows_close(f64(out[b, 0].cpu()), ref["out"][b][0], 2e-2, f"HCA seq {b}")


@pytest.mark.parametrize("cfg", [2, 4, 5])
def test_decode_scores_error_far_inside_the_gap(cfg):
    """Every visible entry's fp32 index score (csa_index_scores, the stage-1 scan of the decode
    workload) against the float64 score: the largest error, relative to the gap rule's scale
    max(|a|, |b|, mean|S|) (a, b the scores ranked K and K + 1, or for the hierarchical
    workload the block maxima ranked 2,048 and 2,049), stays far below half the rule's 1e-3
    margin, so a row that passes the rule ranks the same way in fp32 as in float64."""
    spec = datagen.CONFIGS[cfg]
    case = datagen.make_case(spec)
    q = case["q_idx"].unsqueeze(1).contiguous()
    w = case["w"].unsqueeze(1).contiguous()
    pos = case["pos"].view(-1, 1).contiguous()
    got = csa.index_scores(dev(q), dev(w), dev(case["k_idx"]), dev(pos), spec.m).cpu().numpy()
    worst = 0.0
    for b in range(spec.B):
        n = ocsa.n_visible(int(pos[b, 0]), spec.m, spec.entries)
        s = ocsa.index_scores(f64(case["q_idx"][b]), f64(case["w"][b]), f64(case["k_idx"][b, :n]))
        if spec.block_size:
            ranked = np.sort(np.maximum.reduceat(s, np.arange(0, n, spec.block_size)))[::-1]
            a_, b_ = ranked[spec.max_blocks - 1], ranked[spec.max_blocks]
        else:
            ranked = np.sort(s)[::-1]
            a_, b_ = ranked[spec.K - 1], ranked[spec.K]
        scale = max(abs(a_), abs(b_), np.abs(s).mean())
        worst = max(worst, np.abs(got[b, 0, :n].astype(np.float64) - s).max() / scale)
    print(f"config {cfg}: max |fp32 - exact| / gap scale = {worst:.3e}", flush=True)
    assert worst < 1e-5
