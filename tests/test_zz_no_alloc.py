"""The allocation-free decode step (csa_decode_step_noalloc, the static per-GPU scratch array)
against csa_decode_step with a caller workspace, through the C ABI: two calls in a row on one
GPU, the second with a smaller input, each on its own copy of the same state. Ids must agree
bit for bit and every output row within 2e-2 of the larger magnitude (the attention bar);
the state both calls leave (tails, caches, window rows) must agree exactly."""
import ctypes as C

import numpy as np
import pytest
import torch

import datagen
import sparse_long_context_csa_amd as csa_lib
from sparse_long_context_csa_amd import _lib
from gpu_helpers import assert_rows_close, dev
from oracle.pipeline import f64

pytestmark = pytest.mark.gpu

STATE = ("kv", "k_idx", "x_tail", "z_tail", "xi_tail", "zi_tail")


def _run(case, no_alloc):
    spec = case["spec"]
    g = {k: dev(v) for k, v in case.items() if isinstance(v, torch.Tensor)}
    st = {k: g[k].clone() for k in STATE}
    rings = [dev(r).clone() for r in case["rings"]]
    win_new = [g["x_new"] if (c == 0 and datagen.ring_from_raw(spec)) else None
               for c in range(spec.n_attn)]
    kw = {}
    if spec.block_size:
        kw = dict(block_size=spec.block_size, max_blocks=spec.max_blocks, q_idx2=g["q_idx2"],
                  w2=g["w2"])
    step = csa_lib.DecodeStep(m=spec.m, top_k=spec.K, window=spec.W, scale=case["scale"],
                              pos=g["pos"], x_new=g["x_new"], z_new=g["z_new"],
                              xi_new=g["xi_new"], zi_new=g["zi_new"], bias=g["bias"],
                              bias_i=g["bias_i"], q_idx=g["q_idx"], w=g["w"],
                              q=[dev(x) for x in case["q"]], win=rings, win_new=win_new,
                              sink=[dev(x) for x in case["sink"]], no_alloc=no_alloc,
                              **st, **kw)
    assert (step.ws is None) == no_alloc
    out, idx = step()
    torch.cuda.synchronize()
    return [o.cpu() for o in out], idx.cpu(), {k: v.cpu() for k, v in st.items()}, \
        [r.cpu() for r in rings]


@pytest.mark.parametrize("specs", [[
    # a long-row case (candidate segments, 65,536 entries), then a shorter batch
    datagen.CaseSpec(7300, "decode", B=4, L=262144, m=4, w_cap=128, ragged=True),
    datagen.CaseSpec(7301, "decode", B=2, L=20000, m=4, w_cap=128, ragged=True),
], [
    # the hierarchical step with three attention calls, then a smaller one
    datagen.CaseSpec(7302, "decode", B=3, L=40000, m=1, w_cap=128, block_size=8,
                     max_blocks=512, n_attn=3, ragged=True),
    datagen.CaseSpec(7303, "decode", B=1, L=9000, m=1, w_cap=128, block_size=8,
                     max_blocks=256, n_attn=3, ragged=True),
]], ids=["flat", "hierarchical"])
def test_noalloc_step_matches_decode_step_twice(specs):
    for spec in specs:
        print(f"no-alloc step vs decode step: case {spec.case_id} B={spec.B} L={spec.L}",
              flush=True)
        case = datagen.make_case(spec)
        out_a, idx_a, st_a, rings_a = _run(case, no_alloc=True)
        out_w, idx_w, st_w, rings_w = _run(case, no_alloc=False)
        assert torch.equal(idx_a, idx_w), f"ids differ (case {spec.case_id})"
        for c in range(spec.n_attn):
            for b in range(spec.B):
                assert_rows_close(f64(out_a[c][b]), f64(out_w[c][b]), 2e-2,
                                  f"case {spec.case_id} seq {b} call {c}")
        for k in STATE:
            assert torch.equal(st_a[k], st_w[k]), k
        for ra, rw in zip(rings_a, rings_w):
            assert torch.equal(ra, rw)
        assert any(np.any(o.float().numpy() != 0) for o in out_a)


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    # 16 sequences of 1,048,576 entries need about 80 MiB of workspace: refused on the host
    # before any launch (the descriptor's pointers are never dereferenced)
    spec = datagen.CaseSpec(7304, "decode", B=2, L=4096, m=4, w_cap=128)
    case = datagen.make_case(spec)
    g = {k: dev(v) for k, v in case.items() if isinstance(v, torch.Tensor)}
    d = _lib.DecodeDesc()
    d.dtype, d.m, d.dim, d.n_heads, d.idx_heads, d.idx_dim = 1, 4, 512, 64, 64, 128
    d.top_k, d.window, d.w_cap, d.n_attn, d.n_seq, d.e_cap = 512, 128, 128, 1, 16, 1 << 20
    d.scale = 0.04
    for name in ("pos", "x_new", "z_new", "xi_new", "zi_new", "kv", "k_idx", "x_tail",
                 "z_tail", "xi_tail", "zi_tail", "bias", "bias_i", "q_idx", "w", "out_idx"):
        setattr(d, name, g["x_new"].data_ptr())
    d.q[0] = d.win[0] = d.out[0] = g["x_new"].data_ptr()
    assert csa_lib.lib().csa_decode_step_workspace_size(C.byref(d)) > _lib.NOALLOC_SCRATCH_BYTES
    assert csa_lib.lib().csa_decode_step_noalloc(C.byref(d), None) == -5
