"""Benchmark of the CSA hot path on one MI355X: the fused decode step at 1M context.

Workload (one step = one call of csa_decode_step over the batch): 4 sequences at position
1,048,575 with 262,144 compressed entries each (m = 4); the new token completes a block, so
each step pools one entry per stream, scans all 262,144 indexer keys per sequence (64 heads
x 128), selects the Top-512 and attends over 512 entries + 128 window rows with 64 heads of
dim 512 and a per-head sink. Inputs are seeded synthetic tensors of that shape, resident in
HBM before timing. To keep the 256 MiB Infinity Cache from serving repeat reads, steps
rotate over several independent copies of the per-sequence state (caches, tails, rings).

Prints one JSON line: queries/s (value), the indexer scan's roofline and the float64 oracle
timed on a bounded sample on the host cores. The scan's launch duration comes from HIP events
that the scan kernel's own dispatch takes as its start and stop events (hipExtLaunchKernel), in
every 8th step of the timed region (eager launch; an event-carrying dispatch costs the step
about 4 us more than a plain one, so sampling keeps that out of the headline); with --graph,
from an eager pass of the same length after it.
"""
import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "CSA decode queries/sec at 1M ctx + achieved HBM GB/s and MFMA % of peak"
# the quantised main-cache formats: bytes per entry, metric suffix, config description
KV_ENTRY_BYTES = {"fp8": 576, "fp4": 288}
KV_METRIC = {"fp8": ", FP8 main cache", "fp4": ", FP4 main cache"}
KV_CONFIG = {"fp8": "fp8 (448 E4M3 + 64 bf16 channels, 576 B per entry)",
             "fp4": "fp4 (512 E2M1 + an E4M3 scale per 16 channels, 288 B per entry)"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_threads():
    """Host cores the oracle runs on: the CPUs this process may use (sched_getaffinity), capped
    by OMP_NUM_THREADS when the environment sets it (the share of a shared host), and the BLAS
    library NumPy calls ("openblas", "mkl", ...)."""
    n = len(os.sched_getaffinity(0))
    try:
        n = min(n, int(os.environ["OMP_NUM_THREADS"]))
    except (KeyError, ValueError):
        pass
    vendor = "unknown"
    try:
        from threadpoolctl import threadpool_info
        apis = [i.get("internal_api") for i in threadpool_info() if i.get("user_api") == "blas"]
        vendor = apis[0] if apis else vendor
    except Exception:  # pragma: no cover
        pass
    return max(1, n), vendor


def timed_oracle(fn, budget_s, limit):
    """Run fn(i) for i = 0, 1, ... with BLAS on host_threads() threads until about budget_s
    seconds have passed (at most `limit` calls). Returns (calls, seconds, threads, vendor)."""
    threads, vendor = host_threads()
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=threads, user_api="blas")
    except Exception:  # pragma: no cover
        import contextlib
        ctx = contextlib.nullcontext()
    with ctx:
        done, t0 = 0, time.perf_counter()
        while True:
            fn(done)
            done += 1
            el = time.perf_counter() - t0
            if el >= budget_s or done >= limit:
                break
    return done, el, threads, vendor


def cpu_baseline(case, budget_s):
    """The float64 oracle's decode step, on the host cores, over whole sequences of the same
    workload until about budget_s seconds of work (at most 200 queries)."""
    from oracle import pipeline
    B = case["spec"].B
    done, el, threads, vendor = timed_oracle(
        lambda i: pipeline.decode_step(case, seqs=[i % B]), budget_s, 200)
    return {"value": done / el, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "blas": vendor,
            "sample": f"{done} decode queries (whole sequences of the same workload, each a "
                      f"full step: pool, scan of every visible entry, Top-K, attention) in "
                      f"{el:.1f} s, float64 NumPy, BLAS ({vendor}) on {threads} threads"}


TRAFFIC_FILES = {
    fmt: os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", name)
    for fmt, name in (("bf16", "decode_1m_hbm_traffic.json"),
                      ("mxfp4", "decode_1m_mxfp4_hbm_traffic.json"),
                      ("mxfp4qk", "decode_1m_mxfp4qk_hbm_traffic.json"))}


def source_digest(files) -> str:
    """sha256 over the code of the named kernel sources (package-relative), in order: line
    comments, surrounding blanks and empty lines are dropped, so a comment edit leaves it
    unchanged while any change to the code changes it."""
    h = hashlib.sha256()
    base = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sparse_long_context_csa_amd")
    for f in files:
        with open(os.path.join(base, f), encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def counter_traffic(idx_format="bf16"):
    """HBM bytes per launch of the stage-1 scan from the committed rocprofv3 counter passes
    (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter on a plain copy of known
    size), or None when the kernel's sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILES[idx_format]) as f:
            t = json.load(f)
        if source_digest(t["sources"]) != t["source_sha256"]:
            return None
        return int(t["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def time_prefill_scan(scan, launches: int, warmup: int = 3):
    """The prefill indexer scan alone (``scan``: a csa.IndexScores over the 4,096-query chunk,
    the scan_prefill_kernel launch that csa_index_topk makes for these shapes): `launches`
    calls, each between a pair of HIP events recorded on the stream the library launches on
    (torch's current stream). Returns a roofline dict against the bf16 dense MFMA peak."""
    import torch

    import datagen
    from sparse_long_context_csa_amd import accounting as acc

    spec = datagen.CONFIGS[3]
    for _ in range(warmup):
        scan()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(launches)]
    for a, b in evs:
        a.record()
        scan()
        b.record()
    torch.cuda.synchronize()
    us = [a.elapsed_time(b) * 1e3 for a, b in evs]
    pairs = acc.sum_visible(spec.L - spec.chunk, spec.L, spec.m, spec.entries)
    flops = acc.prefill_indexer_flops(pairs, spec.H_I, spec.d_I)
    avg = sum(us) / len(us)
    tf = flops / (avg * 1e-6) / 1e12
    return {"bound": "mfma", "kernel": "scan_prefill_kernel<12> (indexer scan, chunked prefill)",
            "workload": datagen.WORKLOAD_NAMES[3], "achieved": round(tf, 1), "peak": 2500.0,
            "unit": "TFLOP/s", "frac": round(tf / 2500.0, 4), "flops": flops,
            "visible_pairs": pairs, "avg_launch_us": round(avg, 1),
            "launch_us_min_max": [round(min(us), 1), round(max(us), 1)],
            "timing": f"HIP events on the launch stream around each of {launches} "
                      "csa_index_scores calls (one scan_prefill_kernel launch each, the "
                      "kernel and grid csa_index_topk runs for this chunk)"}


def prefill_scan(dev):
    """The chunked-prefill indexer inputs (drawn as for the prefill workload), the chunk's own
    keys pooled into the cache, and a csa.IndexScores over them."""
    import torch

    import datagen
    import sparse_long_context_csa_amd as csa

    spec = datagen.CONFIGS[3]
    p = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
         for k, v in datagen.make_prefill_indexer(spec).items()}
    e0 = (spec.L - spec.chunk) // spec.m
    csa.compress(p["xi_chunk"], p["zi_chunk"], p["bias_i"], spec.m,
                 out=p["k_idx"][:, e0:e0 + spec.chunk // spec.m],
                 out_seq_stride=spec.entries * spec.d_I)
    return csa.IndexScores(p["q_idx"], p["w"], p["k_idx"], p["q_pos"], spec.m,
                           e_count=p["e_count"])


def prefill_cpu_baseline(case, budget_s):
    """The float64 oracle's chunked prefill (index, Top-K and attention of each query row over
    the cache holding the chunk's entries), on the host cores, over evenly spread query rows
    until about budget_s seconds of work; the chunk's pooling runs once before the clock."""
    from oracle import pipeline
    spec = case["spec"]
    kv_c, ki_c = pipeline.prefill_entries(case)
    per_call = 8
    stride = 97    # coprime with the chunk: rows spread over its whole range
    done, el, threads, vendor = timed_oracle(
        lambda i: pipeline.prefill_rows(
            case, [(0, (i * per_call + j) * stride % spec.chunk) for j in range(per_call)],
            kv_c, ki_c), budget_s, 64)
    rows = done * per_call
    return {"value": rows / el, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "blas": vendor,
            "sample": f"{rows} query rows of the 4,096-query chunk ({per_call} per call, spread "
                      f"over the chunk), each index over every visible entry, Top-K and "
                      f"attention, in {el:.1f} s, float64 NumPy, BLAS ({vendor}) on {threads} "
                      f"threads; the chunk's entries pooled once before timing"}


def bench_prefill(args):
    """Chunked prefill (4,096 queries at the end of a 131,072-token context): pool the
    chunk's 4,096 raw rows into 1,024 entries of both streams, then index + select and
    attend for all 4,096 queries. Reported per chunk, with the indexer call's MFMA rate."""
    import torch

    import datagen
    import sparse_long_context_csa_amd as csa
    from sparse_long_context_csa_amd import accounting as acc

    spec = datagen.CONFIGS[3]
    case = datagen.make_case(spec)
    dev = torch.device("cuda:0")
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in case.items()}
    e0 = (spec.L - spec.chunk) // spec.m
    ne = spec.chunk // spec.m
    E = spec.entries
    copies = max(1, min(args.copies, 2))
    kvs = [g["kv"].clone() for _ in range(copies)]
    kis = [g["k_idx"].clone() for _ in range(copies)]

    c4a = args.compressor == "c4a"
    if c4a:
        # the b-stream rows, logits and bias of both caches (the a stream is the chunk's rows
        # above), and the b rows of the block before the chunk
        cid, tb = spec.case_id, 30
        for nm, d in (("", spec.D), ("i", spec.d_I)):
            g[f"x{nm}b"] = datagen.tensor(cid, tb, (1, spec.chunk, d), "bf16", 1 / math.sqrt(d)).to(dev)
            g[f"z{nm}b"] = datagen.tensor(cid, tb + 1, (1, spec.chunk, d), "bf16", 1.0).to(dev)
            g[f"b{nm}b"] = datagen.tensor(cid, tb + 2, (spec.m, d), "bf16", 0.1).to(dev)
            g[f"x{nm}p"] = datagen.tensor(cid, tb + 3, (1, spec.m, d), "bf16", 1 / math.sqrt(d)).to(dev)
            g[f"z{nm}p"] = datagen.tensor(cid, tb + 4, (1, spec.m, d), "bf16", 1.0).to(dev)
            tb += 5

    def compress_chunk(c):
        if c4a:
            csa.compress_c4a(g["x_chunk"], g["z_chunk"], g["xb"], g["zb"], g["bias"], g["bb"],
                             spec.m, xb_prev=g["xp"], zb_prev=g["zp"],
                             out=kvs[c][:, e0:e0 + ne], out_seq_stride=E * spec.D)
            csa.compress_c4a(g["xi_chunk"], g["zi_chunk"], g["xib"], g["zib"], g["bias_i"],
                             g["bib"], spec.m, xb_prev=g["xip"], zb_prev=g["zip"],
                             out=kis[c][:, e0:e0 + ne], out_seq_stride=E * spec.d_I)
            return
        csa.compress(g["x_chunk"], g["z_chunk"], g["bias"], spec.m, out=kvs[c][:, e0:e0 + ne],
                     out_seq_stride=E * spec.D)
        csa.compress(g["xi_chunk"], g["zi_chunk"], g["bias_i"], spec.m, out=kis[c][:, e0:e0 + ne],
                     out_seq_stride=E * spec.d_I)

    def step(c):
        compress_chunk(c)
        idx = csa.index_topk(g["q_idx"], g["w"], kis[c], g["q_pos"], spec.m, spec.K,
                             e_count=g["e_count"])
        return csa.sparse_attn(g["q"], kvs[c], idx, g["ring"], spec.w_cap, spec.W, g["q_pos"],
                               g["sink"], spec.softmax_scale)

    for i in range(args.warmup):
        step(i % copies)
    torch.cuda.synchronize()
    steps = max(1, min(args.steps, 20))
    t0 = time.perf_counter()
    for i in range(steps):
        step(i % copies)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # phase timing (torch events on the current stream: the library launches on it)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ph = [0.0, 0.0, 0.0]
    for i in range(steps):
        c = i % copies
        evs[0].record()
        compress_chunk(c)
        evs[1].record()
        idx = csa.index_topk(g["q_idx"], g["w"], kis[c], g["q_pos"], spec.m, spec.K,
                             e_count=g["e_count"])
        evs[2].record()
        csa.sparse_attn(g["q"], kvs[c], idx, g["ring"], spec.w_cap, spec.W, g["q_pos"], g["sink"],
                        spec.softmax_scale)
        evs[3].record()
        torch.cuda.synchronize()
        for j in range(3):
            ph[j] += evs[j].elapsed_time(evs[j + 1]) / steps
    pairs = acc.sum_visible(spec.L - spec.chunk, spec.L, spec.m, E)
    flops = acc.prefill_indexer_flops(pairs, spec.H_I, spec.d_I)
    tf = flops / (ph[1] * 1e-3) / 1e12
    ms = wall * 1e3 / steps
    # the scan kernel alone, over the same inputs (copy 0 of the cache, the chunk pooled)
    scan = csa.IndexScores(g["q_idx"], g["w"], kis[0], g["q_pos"], spec.m, e_count=g["e_count"])
    roof = time_prefill_scan(scan, launches=steps)
    roof["traffic"] = None
    del scan
    res = {
        "metric": "CSA chunked-prefill queries/sec (4,096 queries, 131,072 ctx)",
        "value": round(spec.chunk * steps / wall, 1), "unit": "queries/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": datagen.WORKLOAD_NAMES[3], "chunk": spec.chunk, "context": spec.L,
                   "entries": E, "top_k": spec.K, "window": spec.W},
        "roofline": roof,
        "index_topk_call": {"flops": flops, "call_ms": round(ph[1], 4),
                            "tflops_incl_select": round(tf, 1),
                            "frac_incl_select": round(tf / 2500.0, 4)},
        "phases_ms": {"compress": round(ph[0], 4), "index_topk": round(ph[1], 4),
                      "sparse_attn": round(ph[2], 4)},
    }
    # the chunk's compression (both caches): every input row read once, the entries written
    n_in = 4 if c4a else 2
    cbytes = sum(n_in * spec.chunk * d * 2 + (2 * spec.m * d * 2 if c4a else 0)
                 + n_in // 2 * spec.m * d * 2 + ne * d * 2 for d in (spec.D, spec.d_I))
    res["compress"] = {"compressor": args.compressor, "bound": "hbm", "bytes": cbytes,
                       "ms_incl_launches": round(ph[0], 4),
                       "gbs": round(cbytes / (ph[0] * 1e-3) / 1e9, 1)}
    if c4a:
        res["metric"] += ", overlapped two-stream compressor"
        res["config"]["compressor"] = "c4a"
    if not args.no_cpu:
        res["cpu_baseline"] = prefill_cpu_baseline(case, args.cpu_budget)
    print(json.dumps(res), flush=True)


def bench_hca(args):
    """Heavily Compressed Attention decode at 1M context (batch 4, m' = 128, 8,192 entries per
    sequence, no indexer): per step the completed 128-row block of every sequence is pooled
    into its cache (csa_compress) and every query attends densely to all visible entries, the
    window and the sink (csa_sparse_attn with top_k = all). The ring already holds the new
    token's row (prepared before timing), so steps repeat the same work."""
    import torch

    import datagen
    import sparse_long_context_csa_amd as csa

    spec = datagen.HCA_DECODE
    case = datagen.make_case(spec)
    dev = torch.device("cuda:0")
    B, m, E, D, H = spec.B, spec.m, spec.entries, spec.D, spec.H
    pos = case["pos"]
    t = int(pos[0])
    e_new = (t + 1) // m - 1
    copies = max(1, args.copies)
    states = []
    for _ in range(copies):
        xb, zb = case["x_tail"].clone(), case["z_tail"].clone()
        ring = case["rings"][0].clone()
        for b in range(B):
            xb[b, t % m] = case["x_new"][b]
            zb[b, t % m] = case["z_new"][b]
            ring[b, t % spec.w_cap] = case["x_new"][b]
        states.append({"x": xb.to(dev), "z": zb.to(dev), "kv": case["kv"].to(dev),
                       "ring": ring.to(dev)})
    q = case["q"][0].unsqueeze(1).contiguous().to(dev)
    sink = case["sink"][0].to(dev)
    bias = case["bias"].to(dev)
    qp = pos.view(B, 1).to(dev)
    idx = torch.arange(E, dtype=torch.int32).repeat(B, 1, 1).contiguous().to(dev)
    outs = [torch.empty(B, 1, H, D, dtype=torch.bfloat16, device=dev) for _ in range(copies)]
    fp8 = args.kv_format in ("fp8", "fp4")
    quantize = csa.quantize_kv_fp8 if args.kv_format == "fp8" else csa.quantize_kv_fp4
    e_bytes = KV_ENTRY_BYTES.get(args.kv_format, D * 2)
    if fp8:   # the cache as FP8 / FP4 entries; the pooled entry is quantised into it
        for st in states:
            st["kv"] = quantize(st["kv"])
            st["entry"] = torch.empty(B, 1, D, dtype=torch.bfloat16, device=dev)
            st["entry8"] = torch.empty(B, 1, e_bytes, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def step(c, evs=None):
        st = states[c]
        if evs: evs[0].record()
        if fp8:
            csa.compress(st["x"], st["z"], bias, m, out=st["entry"])
            quantize(st["entry"], out=st["entry8"])
            st["kv"][:, e_new:e_new + 1].copy_(st["entry8"])
        else:
            csa.compress(st["x"], st["z"], bias, m, out=st["kv"][:, e_new:], out_seq_stride=E * D)
        if evs: evs[1].record()
        csa.sparse_attn(q, st["kv"], idx, st["ring"], spec.w_cap, spec.W, qp, sink,
                        case["scale"], out=outs[c])
        if evs: evs[2].record()

    for i in range(args.warmup):
        step(i % copies)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i % copies)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n_prof = min(args.steps, 100)
    ph = [0.0, 0.0]
    for i in range(n_prof):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        step(i % copies, evs)
        torch.cuda.synchronize()
        ph[0] += evs[0].elapsed_time(evs[1]) / n_prof
        ph[1] += evs[1].elapsed_time(evs[2]) / n_prof
    attn_bytes = B * (E * e_bytes + spec.W * D * 2) + 2 * B * H * D * 2 + B * E * 4 + H * 4
    comp_bytes = B * (2 * m * D * 2 + D * 2) + m * D * 2
    achieved = attn_bytes / (ph[1] * 1e-3) / 1e9
    res = {
        "metric": "HCA decode queries/sec at 1M ctx (dense attention over 8,192 entries)",
        "value": round(B * args.steps / wall, 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": datagen.WORKLOAD_NAMES[6], "batch": B, "context": spec.L,
                   "m": m, "entries": E, "top_k": "all", "window": spec.W, "heads": H,
                   "head_dim": D, "state_copies": copies},
        "roofline": {"bound": "hbm", "kernel": "attn_dma_kernel + attn_combine_kernel",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_call": attn_bytes,
                     "timing": "torch events around the csa_sparse_attn call (launches included)"},
        "phases_us": {"compress": round(ph[0] * 1e3, 2), "attention": round(ph[1] * 1e3, 2)},
        "compress_bytes": comp_bytes,
    }
    if fp8:
        res["metric"] += KV_METRIC[args.kv_format]
        res["config"]["kv_cache"] = KV_CONFIG[args.kv_format]
    print(json.dumps(res), flush=True)


def bench_norm_rope(args):
    """Per-head RMSNorm + partial RoPE (one fused pass) over a prefill chunk's queries: 4,096
    rows x 64 heads x 512 (256 MiB in, 256 MiB out), positions at the end of a 131,072-token
    context. HBM-bound: reported against 8 TB/s."""
    import torch

    import datagen
    import sparse_long_context_csa_amd as csa

    rows, heads, dim = 4096, 64, 512
    dev = torch.device("cuda:0")
    xs = [datagen.tensor(7, 70 + c, (rows, heads, dim), "bf16", 1.0 / math.sqrt(dim)).to(dev)
          for c in range(2)]
    gamma = datagen.tensor(7, 72, (dim,), "bf16", 0.5).to(dev)
    pos = torch.arange(131072 - rows, 131072, dtype=torch.int64, device=dev)
    outs = [torch.empty_like(x) for x in xs]
    for i in range(args.warmup):
        csa.norm_rope(xs[i % 2], gamma, pos, out=outs[i % 2])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        csa.norm_rope(xs[i % 2], gamma, pos, out=outs[i % 2])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    nbytes = 2 * rows * heads * dim * 2 + dim * 2 + rows * 8
    gbs = nbytes * args.steps / wall / 1e9
    print(json.dumps({
        "metric": "per-head RMSNorm + partial RoPE, one pass (4,096 x 64 x 512 queries)",
        "value": round(rows * args.steps / wall, 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill-chunk queries, 4,096 rows x 64 heads x 512, RoPE on the "
                               "last 64 dims at positions 126,976..131,071",
                   "launch": "eager, back-to-back"},
        "roofline": {"bound": "hbm", "kernel": "norm_rope_kernel", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes_per_launch": nbytes,
                     "timing": "wall clock over back-to-back launches"}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=4, help="state copies rotated across steps")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--scan-event-stride", type=int, default=8,
                    help="time the scan kernel of every n-th timed step with dispatch events")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-prefill-indexer", action="store_true",
                    help="1M decode line: skip its chunked-prefill indexer sub-measurement")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step from a captured HIP graph instead of launching it")
    ap.add_argument("--config", type=int, default=4, choices=(2, 3, 4, 5, 6, 7),
                    help="workload (4: the 1M-context decode headline; 3: chunked prefill; "
                         "6: HCA decode, dense attention over 8,192 entries; 7: the fused "
                         "RMSNorm + RoPE pass over a prefill chunk's queries)")
    ap.add_argument("--idx-format", default="bf16", choices=("bf16", "mxfp4", "mxfp4qk"),
                    help="indexer-key cache of the decode workloads: bf16 keys, or MXFP4 codes "
                         "with one scale byte per 32 channels (csa_quantize_mxfp4 of the same "
                         "keys, made before the timed region); mxfp4qk also takes the indexer "
                         "query into MXFP4 in the scan (FP4 x FP4 products)")
    ap.add_argument("--score-format", default="f32", choices=("f32", "bf16"),
                    help="index scores the selection ranks: fp32, or rounded to bf16 (the "
                         "line then also reports the recall of the fp32 selection)")
    ap.add_argument("--rope-dim", type=int, default=0,
                    help="decode workloads: each query's per-head RMSNorm and RoPE on its last N "
                         "channels (prepared in the selection launch), the completed entry's "
                         "RMSNorm and RoPE before it is stored, and the inverse RoPE on the "
                         "output fused into the attention's store (0: off)")
    ap.add_argument("--kv-format", default="bf16", choices=("bf16", "fp8", "fp4"),
                    help="main KV cache of the decode workloads (--config 2/4/5/6): bf16 "
                         "entries, 576-byte FP8 entries or 288-byte FP4 entries "
                         "(csa_quantize_kv_fp8 / _fp4 of the same entries, made before the "
                         "timed region)")
    ap.add_argument("--compressor", default="single", choices=("single", "c4a"),
                    help="main compressor: the single stream, or the overlapped two-stream "
                         "one (decode workloads 2/4/5: the main entries; chunked prefill, "
                         "--config 3: both caches)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1"}))
        sys.exit(2)

    import torch

    import datagen
    import sparse_long_context_csa_amd as csa
    from sparse_long_context_csa_amd import accounting as acc

    if args.config == 3:
        return bench_prefill(args)
    if args.config == 6:
        return bench_hca(args)
    if args.config == 7:
        return bench_norm_rope(args)
    spec = datagen.CONFIGS[args.config]
    c4a = args.compressor == "c4a"
    if c4a:
        spec = dataclasses.replace(spec, compressor="c4a")
    t0 = time.time()
    case = datagen.make_case(spec)
    log(f"generated inputs in {time.time() - t0:.1f} s")
    dev = torch.device("cuda:0")
    shared = {k: case[k].to(dev) for k in ("pos", "x_new", "z_new", "xi_new", "zi_new", "bias",
                                            "bias_i", "q_idx", "w")
              + (("xb_new", "zb_new", "bias_b") if c4a else ())}
    hier = {}
    if spec.block_size:
        hier = dict(block_size=spec.block_size, max_blocks=spec.max_blocks,
                    q_idx2=case["q_idx2"].to(dev), w2=case["w2"].to(dev))
    qs = [x.to(dev) for x in case["q"]]
    sinks = [x.to(dev) for x in case["sink"]]
    mx = args.idx_format in ("mxfp4", "mxfp4qk")
    qk4 = args.idx_format == "mxfp4qk"
    if mx and (spec.block_size or spec.H_I != 64 or spec.d_I != 128):
        print(json.dumps({"error": "MXFP4 indexer keys: flat 64 x 128 decode workloads only"}))
        sys.exit(2)
    if mx:
        codes, scales = csa.quantize_mxfp4(case["k_idx"].to(dev))
        torch.cuda.synchronize()
    kv8 = None
    if args.kv_format in ("fp8", "fp4"):
        quantize = csa.quantize_kv_fp8 if args.kv_format == "fp8" else csa.quantize_kv_fp4
        kv8 = quantize(case["kv"].to(dev))
        torch.cuda.synchronize()
    q_gammas = None
    kv_gamma = None
    if args.rope_dim:
        q_gammas = [(datagen.tensor(spec.case_id, 90 + c, (spec.D,), spec.dtype, 0.3) + 1.0).to(dev)
                    for c in range(spec.n_attn)]
        kv_gamma = (datagen.tensor(spec.case_id, 95, (spec.D,), spec.dtype, 0.3) + 1.0).to(dev)
    steps_objs, states = [], []
    for c in range(args.copies):
        st = {k: case[k].to(dev) for k in ("kv", "k_idx", "x_tail", "z_tail", "xi_tail", "zi_tail")
              + (("xb_tail", "zb_tail") if c4a else ())}
        if mx:
            st["k_idx"] = codes.clone()
            st["k_idx_scale"] = scales.clone()
        if kv8 is not None:
            st["kv"] = kv8.clone()
        rings = [r.to(dev) for r in case["rings"]]
        win_new = [shared["x_new"] if (i == 0 and datagen.ring_from_raw(spec)) else None
                   for i in range(spec.n_attn)]
        states.append(dict(q=qs, win=rings, win_new=win_new, sink=sinks, **shared, **st, **hier))
        steps_objs.append(csa.DecodeStep(
            m=spec.m, top_k=spec.K, window=spec.W, scale=case["scale"],
            score_format=args.score_format, out_rope_dim=args.rope_dim, q_rope_dim=args.rope_dim,
            q_gamma=q_gammas, kv_gamma=kv_gamma, kv_rope_dim=args.rope_dim,
            compressor=args.compressor, query_fp4=qk4, **states[-1]))
    torch.cuda.synchronize()
    log(f"device state ready: {args.copies} copies, "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated")

    ev = csa.HipEvents()
    n_ev = 5
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        steps_objs[i % args.copies]()
    torch.cuda.synchronize()
    graphs = []
    if args.graph:
        # one HIP graph per state copy: the whole fused step (ingest, scan, select, attention)
        # replays with a single launch
        for st in steps_objs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                st()
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % args.copies].replay()
        torch.cuda.synchronize()

    # timed region: exactly `steps` steps; in eager mode the scan kernel of every
    # `scan_event_stride`-th step takes a pair of HIP events as the start and stop events of
    # its own dispatch (no marker packets)
    stride = max(1, args.scan_event_stride)
    sampled = list(range(args.steps)) if args.graph else list(range(0, args.steps, stride))
    scan_ev = {i: (ev.create(), ev.create()) for i in sampled}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        if graphs:
            graphs[i % args.copies].replay()
        else:
            st = steps_objs[i % args.copies]
            if i in scan_ev:
                st.set_scan_events(*scan_ev[i])
            else:
                st.set_scan_events()
            st()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    if graphs:
        for i in range(args.steps):
            st = steps_objs[i % args.copies]
            st.set_scan_events(*scan_ev[i])
            st()
        torch.cuda.synchronize()
    for st in steps_objs:
        st.set_scan_events()
    scan_launch = [ev.ms(a, b) for a, b in scan_ev.values()]
    for a, b in scan_ev.values():
        ev.destroy(a)
        ev.destroy(b)

    # separate pass: phase boundaries recorded with HIP events (marker packets) on the launch
    # stream; a marker adds its own few microseconds to the phase that follows it
    n_prof = min(args.steps, 100)
    events = [[ev.create() for _ in range(n_ev)] for _ in range(n_prof)]
    for i in range(n_prof):
        st = steps_objs[i % args.copies]
        st.set_events(events[i])
        st()
    torch.cuda.synchronize()
    for st in steps_objs:
        st.set_events([])
    phases = [[ev.ms(e[j], e[j + 1]) for j in range(n_ev - 1)] for e in events]
    for e in events:
        for h in e:
            ev.destroy(h)
    del stream
    if args.calib_copy_mib:
        n = args.calib_copy_mib * 2**20 // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    ms_step = wall * 1e3 / args.steps
    qps = spec.B * args.steps / wall
    mean = [sum(p[j] for p in phases) / len(phases) for j in range(n_ev - 1)]
    scan_ms = sum(scan_launch) / len(scan_launch)
    E = spec.entries
    key_bytes = acc.mxfp4_key_bytes(spec.d_I) if mx else None
    scan_bytes = acc.scan_bytes(spec.B, E, spec.H_I, spec.d_I, key_bytes=key_bytes)
    step_bytes = acc.decode_step_bytes(B=spec.B, n_vis=E, m=spec.m, D=spec.D, H=spec.H,
                                       H_I=spec.H_I, d_I=spec.d_I, K=spec.K, W=spec.W,
                                       n_attn=spec.n_attn,
                                       pool=spec.block_size * spec.max_blocks,
                                       ring_write=datagen.ring_from_raw(spec),
                                       key_bytes=key_bytes,
                                       entry_bytes=KV_ENTRY_BYTES.get(args.kv_format),
                                       c4a=c4a).total
    achieved = scan_bytes / (scan_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": round(qps, 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": datagen.WORKLOAD_NAMES[args.config], "batch": spec.B,
                   "context": spec.L,
                   "entries": E, "m": spec.m, "top_k": spec.K, "window": spec.W,
                   "heads": spec.H, "head_dim": spec.D, "idx_heads": spec.H_I,
                   "idx_dim": spec.d_I, "idx_keys": args.idx_format,
                   "state_copies": args.copies,
                   "launch": "hip_graph" if args.graph else "eager"},
        "roofline": {"bound": "hbm", "kernel": "scan_stream_kernel (indexer scan, stage 1)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (counter_traffic(args.idx_format)
                                 if args.config == 4 and args.idx_format in TRAFFIC_FILES
                                 else None),
                     "avg_launch_us": round(scan_ms * 1e3, 2),
                     "launch_us_min_max": [round(min(scan_launch) * 1e3, 2),
                                           round(max(scan_launch) * 1e3, 2)],
                     "timing": "HIP start/stop events of the scan kernel's own dispatch, "
                               + ("eager pass after the graph-timed region" if graphs else
                                  f"every {stride}th step of the timed region "
                                  f"({len(scan_launch)} launches)"),
                     "algorithmic_bytes_per_launch": scan_bytes},
        "step_hbm": {"algorithmic_bytes": step_bytes,
                     "achieved_gbs": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
                     "frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "phases_us_eager_with_marker_events": {"ingest_compress": round(mean[0] * 1e3, 2), "index_scan": round(mean[1] * 1e3, 2),
                      "select": round(mean[2] * 1e3, 2), "attention": round(mean[3] * 1e3, 2)},
    }
    if args.config != 4:
        res["metric"] = f"CSA decode queries/sec ({datagen.WORKLOAD_NAMES[args.config]})"
    if mx:
        res["metric"] += ", MXFP4 indexer keys" + (" and query" if qk4 else "")
    if kv8 is not None:
        res["metric"] += KV_METRIC[args.kv_format]
        res["config"]["kv_cache"] = KV_CONFIG[args.kv_format]
    if args.rope_dim:
        res["metric"] += (f", query and entry RMSNorm + RoPE and output inverse RoPE on the "
                          f"last {args.rope_dim} channels")
        res["config"]["rope_dim"] = args.rope_dim
    if c4a:
        res["metric"] += ", overlapped two-stream main compressor"
        res["config"]["compressor"] = "c4a"
    if args.score_format == "bf16":
        # recall of the fp32 selection: the same step (idempotent: it rewrites the same tail
        # slot and entry) ranked on fp32 scores, over state copy 0
        ref = csa.DecodeStep(m=spec.m, top_k=spec.K, window=spec.W, scale=case["scale"],
                             score_format="f32", compressor=args.compressor, query_fp4=qk4,
                             **states[0])
        _, ids_bf = steps_objs[0]()
        ids_bf = ids_bf.clone()
        _, ids_f32 = ref()
        torch.cuda.synchronize()
        a, b = ids_bf.cpu().numpy(), ids_f32.cpu().numpy()
        rec = [float(np.isin(b[i][b[i] >= 0], a[i]).mean()) for i in range(spec.B)]
        res["metric"] += ", BF16 index scores"
        res["config"]["scores"] = "bf16"
        res["selection_recall_vs_fp32"] = {"mean": round(float(np.mean(rec)), 5),
                                           "min": round(float(np.min(rec)), 5),
                                           "rows": spec.B}
    if args.config == 4 and not args.no_prefill_indexer:
        # the metric's MFMA share: the chunked-prefill indexer scan, timed in the same run
        res["prefill_indexer"] = time_prefill_scan(prefill_scan(dev), launches=20)
    if not args.no_cpu:
        if mx:
            # the oracle's step with an MXFP4 cache (the new entry's key quantised); the cached
            # keys are scored as generated, which is the same work as scoring their MXFP4 values
            case["idx_format"] = "mxfp4_qk" if qk4 else "mxfp4"
        if kv8 is not None:
            case["kv_format"] = args.kv_format
        if args.rope_dim:
            # the same query, entry and window-row preparation and output inverse RoPE as the
            # GPU step
            case["q_gamma"] = [g.cpu() for g in q_gammas]
            case["kv_gamma"] = kv_gamma.cpu()
            case["q_rope_dim"] = case["kv_rope_dim"] = case["out_rope_dim"] = args.rope_dim
        if args.score_format == "bf16":
            case["score_format"] = "bf16"
        res["cpu_baseline"] = cpu_baseline(case, args.cpu_budget)
        if mx:
            res["cpu_baseline"]["sample"] += (" with an MXFP4 cache (new key quantised; cached "
                                              "keys scored as generated)")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
