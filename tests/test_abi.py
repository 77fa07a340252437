"""The C ABI on the CPU: libcsa loads, exports exactly the functions include/csa.h declares,
the binding's descriptor mirrors the header's struct, and host-side validation rejects bad
calls before anything is launched (none of these calls reaches a kernel)."""
import ctypes as C
import os
import re
import subprocess

import pytest

import sparse_long_context_csa_amd as csa
from sparse_long_context_csa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")


def _header() -> str:
    with open(HEADER) as f:
        text = f.read()
    return re.sub(r"/\*.*?\*/", "", text, flags=re.S)


def declared_functions() -> set[str]:
    return set(re.findall(r"^[A-Za-z_][\w \t]*?\**\s*\b(csa_\w+)\s*\(", _header(), flags=re.M))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_long_context_csa_amd import build
        build.build()
    return _lib.lib()


def test_header_declares_the_calls():
    assert declared_functions() == {
        "csa_abi_version", "csa_status_str", "csa_compress", "csa_index_topk_workspace_size",
        "csa_index_topk", "csa_index_blocks_workspace_size", "csa_index_blocks",
        "csa_sparse_attn_workspace_size", "csa_sparse_attn", "csa_decode_step_workspace_size",
        "csa_decode_step", "csa_quantize_mxfp4", "csa_compress_c4a", "csa_norm_rope",
        "csa_quantize_kv_fp8", "csa_dequantize_kv_fp8", "csa_sparse_attn_fp8",
        "csa_decode_step_noalloc", "csa_index_scores_workspace_size", "csa_index_scores",
        "csa_quantize_kv_fp4", "csa_dequantize_kv_fp4", "csa_sparse_attn_fp4"}


def test_binding_covers_every_declared_function():
    assert set(_lib.SIGNATURES) == declared_functions()


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                        text=True)
    if nm.returncode == 0:
        exported = {ln.split()[-1] for ln in nm.stdout.splitlines()
                    if ln.split() and ln.split()[-1].startswith("csa_")}
        assert exported == declared_functions()


def test_abi_version_and_status_strings(lib):
    m = re.search(r"#define\s+CSA_ABI_VERSION\s+(\d+)", _header())
    assert lib.csa_abi_version() == int(m.group(1))
    for code in _lib.STATUS:
        s = lib.csa_status_str(code)
        assert s and isinstance(s, bytes)
    assert lib.csa_status_str(0) == b"ok"
    assert lib.csa_status_str(12345) == b"unknown status"


def test_decode_desc_mirrors_the_header_struct():
    body = re.search(r"typedef struct csa_decode_desc \{(.*?)\} csa_decode_desc;", _header(),
                     flags=re.S).group(1)
    names = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        for part in decl.split(","):
            nm = re.search(r"(\w+)\s*(\[[^\]]+\])?\s*$", part.strip())
            names.append(nm.group(1))
    assert names == [f[0] for f in _lib.DecodeDesc._fields_]
    m = re.search(r"#define\s+CSA_MAX_ATTN\s+(\d+)", _header())
    assert int(m.group(1)) == _lib.MAX_ATTN
    m = re.search(r"#define\s+CSA_DECODE_EVENTS\s+(\d+)", _header())
    assert int(m.group(1)) == _lib.DECODE_EVENTS
    # natural C layout on x86-64: 12 int32 and 2 int64 (64 B), the float padded to 8 B, then
    # 17 tensor pointers, 5 arrays of CSA_MAX_ATTN pointers, out_idx, the phase events, the
    # scan kernel's start and stop events; idx_format padded to 8 B, k_idx_scale, then
    # score_format, out_rope_dim and rope_base (12 B, padded to 16), the CSA_MAX_ATTN query
    # gammas, q_rope_dim and kv_format (8 B), kv_gamma, kv_rope_dim and compressor (8 B), the
    # b stream's 5 pointers
    n_ptr = 17 + 5 * _lib.MAX_ATTN + 1 + _lib.DECODE_EVENTS + 2
    assert C.sizeof(_lib.DecodeDesc) == (64 + 8 + 8 * n_ptr + 8 + 8 + 16 + 8 * _lib.MAX_ATTN
                                         + 8 + 8 + 8 + 5 * 8)
    for name, val in (("CSA_IDX_DTYPE", _lib.IDX_DTYPE), ("CSA_IDX_MXFP4", _lib.IDX_MXFP4),
                      ("CSA_IDX_MXFP4_QK", _lib.IDX_MXFP4_QK),
                      ("CSA_SCORE_F32", _lib.SCORE_F32), ("CSA_SCORE_BF16", _lib.SCORE_BF16),
                      ("CSA_KV_DTYPE", _lib.KV_DTYPE), ("CSA_KV_FP8", _lib.KV_FP8),
                      ("CSA_KV_FP8_BYTES", _lib.KV_FP8_BYTES), ("CSA_KV_FP4", _lib.KV_FP4),
                      ("CSA_KV_FP4_BYTES", _lib.KV_FP4_BYTES),
                      ("CSA_COMP_SINGLE", _lib.COMP_SINGLE), ("CSA_COMP_C4A", _lib.COMP_C4A)):
        assert int(re.search(rf"#define\s+{name}\s+(\d+)", _header()).group(1)) == val


def test_compress_validation(lib):
    ok = C.c_void_p(16)   # never dereferenced: every call below fails validation or is empty
    assert lib.csa_compress(ok, ok, ok, ok, 1, 8, 0, 64, 4, 7, None) == -3
    assert lib.csa_compress(ok, ok, ok, ok, 1, 8, 0, 64, 0, 1, None) == -2
    assert lib.csa_compress(ok, ok, ok, ok, 1, 256, 0, 64, 129, 1, None) == -2
    assert lib.csa_compress(ok, ok, ok, ok, 1, 9, 0, 64, 4, 1, None) == -2      # n_tok % m
    assert lib.csa_compress(ok, ok, ok, ok, 1, 8, 0, 60, 4, 1, None) == -2      # dim % 8
    assert lib.csa_compress(ok, ok, ok, ok, 1, 8, 64, 64, 4, 1, None) == -2     # stride short
    assert lib.csa_compress(None, ok, ok, ok, 1, 8, 0, 64, 4, 1, None) == -1
    assert lib.csa_compress(None, None, None, None, 0, 8, 0, 64, 4, 1, None) == 0  # empty


def test_index_and_attention_validation(lib):
    ok = C.c_void_p(16)
    args = dict(n_seq=1, n_q=1, e_cap=1024, H=64, d=128, m=4)

    def topk(top_k=512, dtype=1, ws=ok, ws_bytes=1 << 40, q=ok, n_q=1):
        return lib.csa_index_topk(q, ok, ok, ok, None, None, 0, args["n_seq"], n_q,
                                  args["e_cap"], args["H"], args["d"], args["m"], top_k, ok,
                                  None, None, ws, ws_bytes, dtype, None)

    assert topk(dtype=3) == -3
    assert topk(top_k=0) == -2
    assert topk(top_k=4096) == -2
    assert topk(q=None) == -1
    assert topk(ws=None) == -5
    assert topk(ws_bytes=16) == -5
    assert topk(q=None, n_q=0) == 0
    need = lib.csa_index_topk_workspace_size(1, 1, 1024, 512)
    assert need > 1024 * 4 and need % 256 == 0
    assert lib.csa_index_topk_workspace_size(1, 4, 1024, 512) > need
    assert lib.csa_index_blocks_workspace_size(4, 1, 262144, 8, 2048, 0) > 0
    # attention: unknown dtype, window above the ring capacity, missing q
    assert lib.csa_sparse_attn(ok, ok, ok, 512, ok, 128, 128, ok, None, 0.1, ok, 1, 1, 1024,
                               64, 512, ok, 1 << 40, 9, None) == -3
    assert lib.csa_sparse_attn(ok, ok, ok, 512, ok, 64, 128, ok, None, 0.1, ok, 1, 1, 1024,
                               64, 512, ok, 1 << 40, 1, None) == -2      # window > w_cap
    assert lib.csa_sparse_attn(None, ok, ok, 512, ok, 128, 128, ok, None, 0.1, ok, 1, 1, 1024,
                               64, 512, ok, 1 << 40, 1, None) == -1


def _desc(**kw) -> _lib.DecodeDesc:
    d = _lib.DecodeDesc()
    d.dtype, d.m, d.dim, d.n_heads, d.idx_heads, d.idx_dim = 1, 4, 512, 64, 64, 128
    d.top_k, d.window, d.w_cap, d.n_attn, d.n_seq, d.e_cap, d.scale = 512, 128, 128, 1, 4, 4096, 0.04
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_compress_c4a_validation(lib):
    ok = C.c_void_p(16)   # never dereferenced: every call below fails validation or is empty
    def call(xb_prev=None, zb_prev=None, n_tok=8, dim=64, m=4, dtype=1, stride=0, xa=ok):
        return lib.csa_compress_c4a(xa, ok, ok, ok, ok, ok, xb_prev, zb_prev, ok, 1, n_tok,
                                    stride, dim, m, dtype, None)
    assert call(dtype=7) == -3
    assert call(m=0) == -2 and call(m=17) == -2
    assert call(n_tok=9) == -2                     # n_tok % m
    assert call(dim=60) == -2
    assert call(stride=64) == -2                   # stride below 2 entries x 64
    assert call(xb_prev=ok) == -1                  # one previous block pointer without the other
    assert call(xa=None) == -1
    assert lib.csa_compress_c4a(None, None, None, None, None, None, None, None, None, 0, 8, 0,
                                64, 4, 1, None) == 0   # empty


def test_norm_rope_validation(lib):
    ok = C.c_void_p(16)   # never dereferenced: every call below fails validation or is empty
    def call(dim=512, rope=64, base=1e4, eps=1e-6, flags=3, dtype=1, gamma=ok, pos=ok, n=2):
        return lib.csa_norm_rope(ok, gamma, pos, ok, n, 64, dim, rope, base, eps, flags, dtype,
                                 None)
    assert call(dtype=5) == -3
    assert call(dim=520) == -2 and call(dim=12) == -2
    assert call(rope=63) == -2 and call(rope=600) == -2
    assert call(base=1.0) == -2 and call(eps=-1.0) == -2 and call(flags=8) == -2
    assert call(flags=5) == -2                     # inverse without RoPE
    assert call(gamma=None) == -1 and call(pos=None) == -1
    assert call(n=0) == 0


def test_quantize_mxfp4_validation(lib):
    ok = C.c_void_p(16)   # never dereferenced: every call below fails validation or is empty
    assert lib.csa_quantize_mxfp4(ok, ok, ok, 4, 128, 7, None) == -3       # dtype
    assert lib.csa_quantize_mxfp4(ok, ok, ok, 4, 100, 1, None) == -2       # dim % 32
    assert lib.csa_quantize_mxfp4(ok, ok, ok, -1, 128, 1, None) == -2
    assert lib.csa_quantize_mxfp4(None, ok, ok, 4, 128, 1, None) == -1
    assert lib.csa_quantize_mxfp4(ok, ok, ok, 0, 128, 1, None) == 0        # nothing to do


def test_kv_fp8_validation(lib):
    ok = C.c_void_p(256)   # never dereferenced: every call below fails validation or is empty
    assert lib.csa_quantize_kv_fp8(ok, ok, 4, 7, None) == -3             # dtype
    assert lib.csa_quantize_kv_fp8(ok, ok, -1, 1, None) == -2
    assert lib.csa_quantize_kv_fp8(None, ok, 4, 1, None) == -1
    assert lib.csa_quantize_kv_fp8(ok, C.c_void_p(256 + 8), 4, 1, None) == -2   # alignment
    assert lib.csa_quantize_kv_fp8(ok, ok, 0, 1, None) == 0              # nothing to do
    assert lib.csa_dequantize_kv_fp8(ok, None, 4, None) == -1
    assert lib.csa_dequantize_kv_fp8(C.c_void_p(256 + 4), ok, 4, None) == -2
    assert lib.csa_dequantize_kv_fp8(ok, ok, -3, None) == -2
    assert lib.csa_dequantize_kv_fp8(ok, ok, 0, None) == 0

    def attn(kv=ok, H=64, D=512, dtype=1):
        return lib.csa_sparse_attn_fp8(ok, kv, ok, 512, ok, 128, 128, ok, None, 0.1, ok, 1, 1,
                                       1024, H, D, ok, 1 << 40, dtype, None)

    assert attn(dtype=0) == -4            # the FP8 cache is read by the bf16 64 x 512 path
    assert attn(H=32) == -4
    assert attn(D=256) == -4
    assert attn(dtype=9) == -3
    assert attn(kv=C.c_void_p(256 + 8)) == -2


def test_kv_fp4_validation(lib):
    ok = C.c_void_p(256)   # never dereferenced: every call below fails validation or is empty
    assert lib.csa_quantize_kv_fp4(ok, ok, 4, 7, None) == -3             # dtype
    assert lib.csa_quantize_kv_fp4(ok, ok, -1, 1, None) == -2
    assert lib.csa_quantize_kv_fp4(None, ok, 4, 1, None) == -1
    assert lib.csa_quantize_kv_fp4(ok, C.c_void_p(256 + 8), 4, 1, None) == -2   # alignment
    assert lib.csa_quantize_kv_fp4(ok, ok, 0, 1, None) == 0              # nothing to do
    assert lib.csa_dequantize_kv_fp4(ok, None, 4, None) == -1
    assert lib.csa_dequantize_kv_fp4(C.c_void_p(256 + 4), ok, 4, None) == -2
    assert lib.csa_dequantize_kv_fp4(ok, C.c_void_p(256 + 8), 4, None) == -2
    assert lib.csa_dequantize_kv_fp4(ok, ok, -3, None) == -2
    assert lib.csa_dequantize_kv_fp4(ok, ok, 0, None) == 0

    def attn(kv=ok, H=64, D=512, dtype=1):
        return lib.csa_sparse_attn_fp4(ok, kv, ok, 512, ok, 128, 128, ok, None, 0.1, ok, 1, 1,
                                       1024, H, D, ok, 1 << 40, dtype, None)

    assert attn(dtype=0) == -4            # the FP4 cache is read by the bf16 64 x 512 path
    assert attn(H=32) == -4
    assert attn(D=256) == -4
    assert attn(dtype=9) == -3
    assert attn(kv=C.c_void_p(256 + 8)) == -2


def test_index_scores_validation(lib):
    ok = C.c_void_p(256)   # never dereferenced: every call below fails validation or is empty
    nb = lib.csa_index_scores_workspace_size(2, 1, 1000)
    assert nb > 0 and lib.csa_index_scores_workspace_size(2, 1, 0) == 0

    def call(scores=ok, stride=1000, e_cap=1000, ws=ok, ws_bytes=nb, dtype=1, q=ok, n_seq=2):
        return lib.csa_index_scores(q, ok, ok, ok, None, n_seq, 1, e_cap, 64, 128, 4, scores,
                                    stride, ws, ws_bytes, dtype, None)
    assert call(dtype=7) == -3
    assert call(stride=996) == -2                   # below e_cap
    assert call(stride=1002) == -2                  # not a multiple of 4
    assert call(scores=C.c_void_p(256 + 4)) == -2   # rows not 16-byte aligned
    assert call(q=None) == -1
    assert call(ws_bytes=nb - 1) == -5
    assert call(ws=None) == -5
    assert call(n_seq=0) == 0


def test_decode_validation(lib):
    d = _desc()
    nb = lib.csa_decode_step_workspace_size(C.byref(d))
    assert nb > 0 and nb % 256 == 0
    assert lib.csa_decode_step(C.byref(d), C.c_void_p(16), nb, None) == -1   # null tensors
    assert lib.csa_decode_step(None, None, 0, None) == -1
    assert lib.csa_decode_step(C.byref(_desc(n_attn=5)), C.c_void_p(16), nb, None) == -2
    assert lib.csa_decode_step(C.byref(_desc(dtype=4)), C.c_void_p(16), nb, None) == -3
    assert lib.csa_decode_step_workspace_size(C.byref(_desc(top_k=0))) == 0
    assert lib.csa_decode_step(C.byref(_desc(n_seq=0)), None, 0, None) == 0
    # hierarchical pools above 32,768 entries are outside the limits
    big = _desc(block_size=64, max_blocks=1024)
    assert lib.csa_decode_step(C.byref(big), C.c_void_p(16), nb, None) == -4
    # every pointer set (never dereferenced): one scan event without the other is refused
    # before anything is launched
    full = _desc()
    for name, typ in _lib.DecodeDesc._fields_:
        if typ is C.c_void_p:
            setattr(full, name, 16)
        elif name in ("q", "win", "win_new", "sink", "out"):
            getattr(full, name)[0] = 16
    full.scan_events[0] = 16
    assert lib.csa_decode_step(C.byref(full), C.c_void_p(16), nb, None) == -1
    full.scan_events[0] = 0


def test_decode_noalloc_validation(lib):
    # the allocation-free step validates like csa_decode_step, and refuses a step whose
    # workspace exceeds the static scratch before touching the GPU
    assert lib.csa_decode_step_noalloc(None, None) == -1
    assert lib.csa_decode_step_noalloc(C.byref(_desc(n_attn=5)), None) == -2
    assert lib.csa_decode_step_noalloc(C.byref(_desc(n_seq=0)), None) == 0
    full = _desc(n_seq=16, e_cap=1 << 20)
    nb = lib.csa_decode_step_workspace_size(C.byref(full))
    assert nb > _lib.NOALLOC_SCRATCH_BYTES
    for name, typ in _lib.DecodeDesc._fields_:
        if typ is C.c_void_p and name not in ("k_idx_scale", "kv_gamma"):
            setattr(full, name, 16)
        elif name in ("q", "win", "win_new", "sink", "out"):
            getattr(full, name)[0] = 16
    full.scan_events[0] = full.scan_events[1] = 0
    for i in range(_lib.DECODE_EVENTS):
        full.events[i] = 0
    assert lib.csa_decode_step_noalloc(C.byref(full), None) == -5
    hdr = re.search(r"#define\s+CSA_NOALLOC_SCRATCH_BYTES\s+\((\d+)u << (\d+)\)", _header())
    assert int(hdr.group(1)) << int(hdr.group(2)) == _lib.NOALLOC_SCRATCH_BYTES


def test_decode_compressor_validation(lib):
    # the overlapped compressor needs the b stream's five pointers; an unknown compressor is a
    # shape error; both refused before anything is launched
    d = _desc(compressor=_lib.COMP_C4A)
    for name, typ in _lib.DecodeDesc._fields_:
        if typ is C.c_void_p and name not in ("k_idx_scale", "kv_gamma"):
            setattr(d, name, 256)
        elif name in ("q", "win", "win_new", "sink", "out"):
            getattr(d, name)[0] = 256
    d.scan_events[0] = d.scan_events[1] = None
    for i in range(_lib.DECODE_EVENTS):
        d.events[i] = None
    nb = lib.csa_decode_step_workspace_size(C.byref(d))
    assert nb > 0
    for name in ("xb_new", "zb_new", "xb_tail", "zb_tail", "bias_b"):
        keep = getattr(d, name)
        setattr(d, name, None)
        assert lib.csa_decode_step(C.byref(d), C.c_void_p(256), nb, None) == -1, name
        assert lib.csa_decode_step_noalloc(C.byref(d), None) == -1, name
        setattr(d, name, keep)
    d.compressor = 2
    assert lib.csa_decode_step(C.byref(d), C.c_void_p(256), nb, None) == -2
    assert lib.csa_decode_step_workspace_size(C.byref(d)) == 0


def test_decode_mxfp4_validation(lib):
    def full(**kw):
        d = _desc(**{"idx_format": _lib.IDX_MXFP4, **kw})
        for name, typ in _lib.DecodeDesc._fields_:
            if typ is C.c_void_p:
                setattr(d, name, 256)
            elif name in ("q", "win", "win_new", "sink", "out"):
                getattr(d, name)[0] = 256
        d.scan_events[0] = d.scan_events[1] = None
        for i in range(_lib.DECODE_EVENTS):
            d.events[i] = None
        return d

    nb = lib.csa_decode_step_workspace_size(C.byref(_desc()))
    ws = C.c_void_p(256)

    def step(d):
        return lib.csa_decode_step(C.byref(d), ws, nb, None)

    # every call below is refused before anything is launched
    assert step(full(idx_format=3)) == -2
    for fmt in (_lib.IDX_MXFP4, _lib.IDX_MXFP4_QK):          # keys alone, or keys and query
        assert step(full(idx_format=fmt, block_size=8, max_blocks=64)) == -4   # hierarchical
        assert step(full(idx_format=fmt, m=16)) == -4         # the scan pools m <= 8 only
        assert step(full(idx_format=fmt, idx_dim=64)) == -4
        assert step(full(idx_format=fmt, dtype=0)) == -4      # fp32 step
        d = full(idx_format=fmt)
        d.k_idx_scale = None
        assert step(d) == -1
        d = full(idx_format=fmt)
        d.k_idx = 256 + 8                                     # codes not 16-byte aligned
        assert step(d) == -2
        d = full(idx_format=fmt)
        d.k_idx_scale = 256 + 2
        assert step(d) == -2
    assert lib.csa_decode_step_workspace_size(C.byref(full(m=16))) == 0
    # BF16 scores: flat selection and the stream scan's shapes only
    d = full(idx_format=_lib.IDX_DTYPE, score_format=_lib.SCORE_BF16, block_size=8,
             max_blocks=64)
    assert step(d) == -4
    assert step(full(idx_format=_lib.IDX_DTYPE, score_format=_lib.SCORE_BF16, idx_dim=64)) == -4
    assert step(full(idx_format=_lib.IDX_DTYPE, score_format=3)) == -2
    # inverse RoPE on the output: even, within dim, a multiple of 16 on the 64 x 512 path
    assert step(full(idx_format=_lib.IDX_DTYPE, out_rope_dim=63, rope_base=1e4)) == -2
    assert step(full(idx_format=_lib.IDX_DTYPE, out_rope_dim=600, rope_base=1e4)) == -2
    assert step(full(idx_format=_lib.IDX_DTYPE, out_rope_dim=64, rope_base=1.0)) == -2
    assert step(full(idx_format=_lib.IDX_DTYPE, out_rope_dim=40, rope_base=1e4)) == -4
    assert step(full(idx_format=_lib.IDX_DTYPE, q_rope_dim=7, rope_base=1e4)) == -2
    assert step(full(idx_format=_lib.IDX_DTYPE, q_rope_dim=64, rope_base=0.5)) == -2
    # FP8 / FP4 main cache: bf16 64 x 512 heads, 16-byte aligned entries, a known format code
    assert step(full(idx_format=_lib.IDX_DTYPE, kv_format=3)) == -2
    for fmt in (_lib.KV_FP8, _lib.KV_FP4):
        assert step(full(idx_format=_lib.IDX_DTYPE, kv_format=fmt, dtype=0)) == -4
        assert step(full(idx_format=_lib.IDX_DTYPE, kv_format=fmt, n_heads=32)) == -4
        d = full(idx_format=_lib.IDX_DTYPE, kv_format=fmt)
        d.kv = 256 + 8
        assert step(d) == -2
    # the new entry's RMSNorm / RoPE: 512-channel entries, even kv_rope_dim <= 64, a base > 1
    assert step(full(idx_format=_lib.IDX_DTYPE, kv_rope_dim=7)) == -2
    assert step(full(idx_format=_lib.IDX_DTYPE, kv_rope_dim=64, rope_base=1.0)) == -2
    assert step(full(idx_format=_lib.IDX_DTYPE, kv_rope_dim=128, rope_base=1e4)) == -4
    assert step(full(idx_format=_lib.IDX_DTYPE, kv_gamma=256, dim=256)) == -4


def test_binding_raises_on_errors(lib):
    with pytest.raises(_lib.CsaError) as e:
        _lib.check("csa_compress", -2)
    assert "CSA_ERR_SHAPE" in str(e.value)
    assert csa.lib() is lib
