"""ctypes loader of libcsa.so: the C ABI of include/csa.h, symbol for symbol."""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LIBCSA_PATH", os.path.join(_HERE, "libcsa.so"))

CSA_F32, CSA_BF16 = 0, 1
STATUS = {0: "CSA_OK", -1: "CSA_ERR_NULL", -2: "CSA_ERR_SHAPE", -3: "CSA_ERR_DTYPE",
          -4: "CSA_ERR_UNSUPPORTED", -5: "CSA_ERR_WORKSPACE", -6: "CSA_ERR_HIP"}
MAX_ATTN = 4
DECODE_EVENTS = 5
IDX_DTYPE, IDX_MXFP4, IDX_MXFP4_QK = 0, 1, 2
SCORE_F32, SCORE_BF16 = 0, 1
KV_DTYPE, KV_FP8, KV_FP4 = 0, 1, 2
KV_FP8_BYTES = 576
KV_FP4_BYTES = 288
NOALLOC_SCRATCH_BYTES = 32 << 20
NR_NORM, NR_ROPE, NR_INVERSE = 1, 2, 4
COMP_SINGLE, COMP_C4A = 0, 1

vp, i32, i64, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t


class DecodeDesc(C.Structure):
    """Mirror of csa_decode_desc (include/csa.h)."""
    _fields_ = [
        ("dtype", i32), ("m", i32), ("dim", i32), ("n_heads", i32), ("idx_heads", i32),
        ("idx_dim", i32), ("top_k", i32), ("window", i32), ("w_cap", i32),
        ("block_size", i32), ("max_blocks", i32), ("n_attn", i32),
        ("n_seq", i64), ("e_cap", i64), ("scale", f32),
        ("pos", vp), ("x_new", vp), ("z_new", vp), ("xi_new", vp), ("zi_new", vp),
        ("kv", vp), ("k_idx", vp), ("x_tail", vp), ("z_tail", vp), ("xi_tail", vp),
        ("zi_tail", vp), ("bias", vp), ("bias_i", vp), ("q_idx", vp), ("w", vp),
        ("q_idx2", vp), ("w2", vp), ("q", vp * MAX_ATTN), ("win", vp * MAX_ATTN),
        ("win_new", vp * MAX_ATTN), ("sink", vp * MAX_ATTN), ("out", vp * MAX_ATTN),
        ("out_idx", vp), ("events", vp * DECODE_EVENTS), ("scan_events", vp * 2),
        ("idx_format", i32), ("k_idx_scale", vp), ("score_format", i32),
        ("out_rope_dim", i32), ("rope_base", f32),
        ("q_gamma", vp * MAX_ATTN), ("q_rope_dim", i32), ("kv_format", i32),
        ("kv_gamma", vp), ("kv_rope_dim", i32),
        ("compressor", i32), ("xb_new", vp), ("zb_new", vp), ("xb_tail", vp), ("zb_tail", vp),
        ("bias_b", vp),
    ]


SIGNATURES = {
    "csa_abi_version": (i32, []),
    "csa_status_str": (C.c_char_p, [i32]),
    "csa_compress": (i32, [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, vp]),
    "csa_compress_c4a": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, vp]),
    "csa_norm_rope": (i32, [vp, vp, vp, vp, i64, i32, i32, i32, f32, f32, i32, i32, vp]),
    "csa_quantize_mxfp4": (i32, [vp, vp, vp, i64, i32, i32, vp]),
    "csa_quantize_kv_fp8": (i32, [vp, vp, i64, i32, vp]),
    "csa_dequantize_kv_fp8": (i32, [vp, vp, i64, vp]),
    "csa_quantize_kv_fp4": (i32, [vp, vp, i64, i32, vp]),
    "csa_dequantize_kv_fp4": (i32, [vp, vp, i64, vp]),
    "csa_index_topk_workspace_size": (sz, [i64, i64, i64, i32]),
    "csa_index_scores_workspace_size": (sz, [i64, i64, i64]),
    "csa_index_scores": (i32, [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, vp, i64, vp, sz,
                              i32, vp]),
    "csa_index_topk": (i32, [vp, vp, vp, vp, vp, vp, i32, i64, i64, i64, i32, i32, i32, i32,
                             vp, vp, vp, vp, sz, i32, vp]),
    "csa_index_blocks_workspace_size": (sz, [i64, i64, i64, i32, i32, i32]),
    "csa_index_blocks": (i32, [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32, i32, vp,
                               i32, vp, vp, sz, i32, vp]),
    "csa_sparse_attn_workspace_size": (sz, [i64, i64, i32, i32, i32, i32]),
    "csa_sparse_attn": (i32, [vp, vp, vp, i32, vp, i32, i32, vp, vp, f32, vp, i64, i64, i64,
                              i32, i32, vp, sz, i32, vp]),
    "csa_sparse_attn_fp8": (i32, [vp, vp, vp, i32, vp, i32, i32, vp, vp, f32, vp, i64, i64,
                                  i64, i32, i32, vp, sz, i32, vp]),
    "csa_sparse_attn_fp4": (i32, [vp, vp, vp, i32, vp, i32, i32, vp, vp, f32, vp, i64, i64,
                                  i64, i32, i32, vp, sz, i32, vp]),
    "csa_decode_step_workspace_size": (sz, [C.POINTER(DecodeDesc)]),
    "csa_decode_step": (i32, [C.POINTER(DecodeDesc), vp, sz, vp]),
    "csa_decode_step_noalloc": (i32, [C.POINTER(DecodeDesc), vp]),
}

_lib = None


def lib() -> C.CDLL:
    """The loaded libcsa (raises if it has not been built: there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libcsa is not built ({LIB_PATH} missing): run "
                               "`python -m sparse_long_context_csa_amd.build` first")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


class CsaError(RuntimeError):
    def __init__(self, call: str, status: int):
        msg = lib().csa_status_str(status).decode()
        super().__init__(f"{call} failed: {STATUS.get(status, status)} ({msg})")
        self.status = status


def check(call: str, status: int) -> None:
    if status != 0:
        raise CsaError(call, status)
