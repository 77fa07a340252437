"""Python binding of libcsa, the CSA hot path for MI355X (gfx950).

Argument marshalling only: every step runs in libcsa's HIP kernels. PyTorch provides
device memory (tensors, workspaces) and the current HIP stream. The functions mirror the
C ABI of include/csa.h; see there for the exact contract of each call.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _lib
from ._events import HipEvents  # noqa: F401
from ._lib import CsaError, DecodeDesc, check, lib  # noqa: F401

__all__ = ["compress", "index_topk", "index_scores", "IndexScores", "index_blocks", "sparse_attn", "DecodeStep", "CsaError",
           "lib"]


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.CSA_BF16
    if t.dtype == torch.float32:
        return _lib.CSA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _dev(t, name: str, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _p(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------------------
def compress(x: torch.Tensor, logits: torch.Tensor, bias: torch.Tensor, m: int,
             out: torch.Tensor | None = None, out_seq_stride: int = 0) -> torch.Tensor:
    """csa_compress: pool every m rows of x [n_seq, n_tok, dim] into one entry."""
    _dev(x, "x"); _dev(logits, "logits", x.dtype); _dev(bias, "bias", x.dtype)
    n_seq, n_tok, dim = x.shape
    if out is None:
        out = torch.empty(n_seq, n_tok // m, dim, dtype=x.dtype, device=x.device)
    elif out.dtype != x.dtype or not out.is_cuda:
        raise TypeError("out must be a GPU tensor of x's dtype")
    check("csa_compress", lib().csa_compress(_p(x), _p(logits), _p(bias), _p(out), n_seq, n_tok,
                                             out_seq_stride, dim, m, _dtype(x), _stream()))
    return out


def compress_c4a(xa: torch.Tensor, za: torch.Tensor, xb: torch.Tensor, zb: torch.Tensor,
                 bias_a: torch.Tensor, bias_b: torch.Tensor, m: int, xb_prev=None, zb_prev=None,
                 out: torch.Tensor | None = None, out_seq_stride: int = 0) -> torch.Tensor:
    """csa_compress_c4a: rows [n_seq, n_tok, dim] of both streams -> entries [n_seq, n_tok/m,
    dim]; xb_prev/zb_prev [n_seq, m, dim] the b rows of the block before the chunk, or None at
    the start of a sequence."""
    for nm, t in (("xa", xa), ("za", za), ("xb", xb), ("zb", zb), ("bias_a", bias_a),
                  ("bias_b", bias_b)):
        _dev(t, nm, xa.dtype)
    _dev(xb_prev, "xb_prev", xa.dtype); _dev(zb_prev, "zb_prev", xa.dtype)
    n_seq, n_tok, dim = xa.shape
    for t in (za, xb, zb):
        if tuple(t.shape) != (n_seq, n_tok, dim):
            raise ValueError("xa, za, xb and zb must have the same shape")
    if out is None:
        out = torch.empty(n_seq, n_tok // m, dim, dtype=xa.dtype, device=xa.device)
    check("csa_compress_c4a", lib().csa_compress_c4a(
        _p(xa), _p(za), _p(xb), _p(zb), _p(bias_a), _p(bias_b), _p(xb_prev), _p(zb_prev),
        _p(out), n_seq, n_tok, out_seq_stride, dim, m, _dtype(xa), _stream()))
    return out


def norm_rope(x: torch.Tensor, gamma: torch.Tensor | None = None,
              pos: torch.Tensor | None = None, rope_dim: int = 64, rope_base: float = 10000.0,
              eps: float = 1e-6, inverse: bool = False, out: torch.Tensor | None = None):
    """csa_norm_rope over x [n_rows, n_heads, dim]: RMSNorm when gamma [dim] is given, RoPE on
    the last rope_dim channels when pos [n_rows] (i64) is given (at -pos with inverse)."""
    _dev(x, "x"); _dev(gamma, "gamma", x.dtype); _dev(pos, "pos", torch.int64)
    n_rows, n_heads, dim = x.shape
    flags = (_lib.NR_NORM if gamma is not None else 0) | (_lib.NR_ROPE if pos is not None else 0)
    if inverse:
        flags |= _lib.NR_INVERSE
    if out is None:
        out = torch.empty_like(x)
    check("csa_norm_rope", lib().csa_norm_rope(_p(x), _p(gamma), _p(pos), _p(out), n_rows, n_heads,
                                               dim, rope_dim, float(rope_base), float(eps), flags,
                                               _dtype(x), _stream()))
    return out


def quantize_mxfp4(x: torch.Tensor, codes: torch.Tensor | None = None,
                   scales: torch.Tensor | None = None):
    """csa_quantize_mxfp4: rows x [..., dim] -> (codes uint8 [..., dim/2], scales uint8 [..., dim/32])."""
    _dev(x, "x")
    dim = x.shape[-1]
    n_rows = x.numel() // dim if dim else 0
    if codes is None:
        codes = torch.empty(*x.shape[:-1], dim // 2, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(*x.shape[:-1], dim // 32, dtype=torch.uint8, device=x.device)
    _dev(codes, "codes", torch.uint8)
    _dev(scales, "scales", torch.uint8)
    check("csa_quantize_mxfp4", lib().csa_quantize_mxfp4(_p(x), _p(codes), _p(scales), n_rows, dim,
                                                         _dtype(x), _stream()))
    return codes, scales


def quantize_kv_fp8(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """csa_quantize_kv_fp8: entries x [..., 512] -> FP8 entries uint8 [..., 576]."""
    _dev(x, "x")
    if x.shape[-1] != 512:
        raise ValueError("FP8 entries are 512 channels wide")
    n_rows = x.numel() // 512
    if out is None:
        out = torch.empty(*x.shape[:-1], _lib.KV_FP8_BYTES, dtype=torch.uint8, device=x.device)
    _dev(out, "out", torch.uint8)
    check("csa_quantize_kv_fp8", lib().csa_quantize_kv_fp8(_p(x), _p(out), n_rows, _dtype(x),
                                                           _stream()))
    return out


def dequantize_kv_fp8(e: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """csa_dequantize_kv_fp8: FP8 entries uint8 [..., 576] -> bf16 [..., 512]."""
    _dev(e, "e", torch.uint8)
    if e.shape[-1] != _lib.KV_FP8_BYTES:
        raise ValueError("FP8 entries are 576 bytes")
    n_rows = e.numel() // _lib.KV_FP8_BYTES
    if out is None:
        out = torch.empty(*e.shape[:-1], 512, dtype=torch.bfloat16, device=e.device)
    _dev(out, "out", torch.bfloat16)
    check("csa_dequantize_kv_fp8", lib().csa_dequantize_kv_fp8(_p(e), _p(out), n_rows, _stream()))
    return out


def quantize_kv_fp4(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """csa_quantize_kv_fp4: entries x [..., 512] -> FP4 entries uint8 [..., 288]."""
    _dev(x, "x")
    if x.shape[-1] != 512:
        raise ValueError("FP4 entries are 512 channels wide")
    n_rows = x.numel() // 512
    if out is None:
        out = torch.empty(*x.shape[:-1], _lib.KV_FP4_BYTES, dtype=torch.uint8, device=x.device)
    _dev(out, "out", torch.uint8)
    check("csa_quantize_kv_fp4", lib().csa_quantize_kv_fp4(_p(x), _p(out), n_rows, _dtype(x),
                                                           _stream()))
    return out


def dequantize_kv_fp4(e: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """csa_dequantize_kv_fp4: FP4 entries uint8 [..., 288] -> bf16 [..., 512]."""
    _dev(e, "e", torch.uint8)
    if e.shape[-1] != _lib.KV_FP4_BYTES:
        raise ValueError("FP4 entries are 288 bytes")
    n_rows = e.numel() // _lib.KV_FP4_BYTES
    if out is None:
        out = torch.empty(*e.shape[:-1], 512, dtype=torch.bfloat16, device=e.device)
    _dev(out, "out", torch.bfloat16)
    check("csa_dequantize_kv_fp4", lib().csa_dequantize_kv_fp4(_p(e), _p(out), n_rows, _stream()))
    return out


def _kv_entry_format(kv) -> int:
    """KV_DTYPE, or the quantised format a uint8 kv holds, told by its entry width."""
    if kv is None or kv.dtype != torch.uint8:
        return _lib.KV_DTYPE
    if kv.shape[-1] == _lib.KV_FP8_BYTES:
        return _lib.KV_FP8
    if kv.shape[-1] == _lib.KV_FP4_BYTES:
        return _lib.KV_FP4
    raise ValueError("a uint8 kv holds 576-byte FP8 or 288-byte FP4 entries")


def index_topk(q_idx: torch.Tensor, w: torch.Tensor, k_idx: torch.Tensor, q_pos: torch.Tensor,
               m: int, top_k: int, e_count: torch.Tensor | None = None,
               cand: torch.Tensor | None = None, want_scores: bool = False,
               want_all: bool = False):
    """csa_index_topk. q_idx [n_seq,n_q,H_I,d_I], w [n_seq,n_q,H_I] f32, k_idx [n_seq,e_cap,d_I],
    q_pos [n_seq,n_q] i64, optional e_count [n_seq] i32 and cand [n_seq,n_q,n_cand] i32.
    Returns out_idx (and out_score / scores_all when asked)."""
    _dev(q_idx, "q_idx"); _dev(w, "w", torch.float32); _dev(k_idx, "k_idx", q_idx.dtype)
    _dev(q_pos, "q_pos", torch.int64); _dev(e_count, "e_count", torch.int32)
    _dev(cand, "cand", torch.int32)
    n_seq, n_q, H, d = q_idx.shape
    e_cap = k_idx.shape[1]
    n_cand = 0 if cand is None else cand.shape[-1]
    n_keys = n_cand if cand is not None else e_cap
    dev = q_idx.device
    out_idx = torch.empty(n_seq, n_q, top_k, dtype=torch.int32, device=dev)
    out_score = torch.empty(n_seq, n_q, top_k, dtype=torch.float32, device=dev) if want_scores else None
    all_s = torch.empty(n_seq, n_q, n_keys, dtype=torch.float32, device=dev) if want_all else None
    nb = lib().csa_index_topk_workspace_size(n_seq, n_q, n_keys, top_k)
    ws = _workspace(nb, dev)
    check("csa_index_topk", lib().csa_index_topk(
        _p(q_idx), _p(w), _p(k_idx), _p(q_pos), _p(e_count), _p(cand), n_cand, n_seq, n_q, e_cap,
        H, d, m, top_k, _p(out_idx), _p(out_score), _p(all_s), _p(ws), ws.numel(), _dtype(q_idx),
        _stream()))
    res = [out_idx]
    if want_scores:
        res.append(out_score)
    if want_all:
        res.append(all_s)
    return res[0] if len(res) == 1 else tuple(res)


class IndexScores:
    """csa_index_scores over fixed inputs: builds the output rows (stride e_cap rounded up to a
    multiple of 4 floats) and the workspace once; each call scores every visible entry of
    every query row on the current stream. q_idx [n_seq,n_q,H_I,d_I], w [n_seq,n_q,H_I] f32,
    k_idx [n_seq,e_cap,d_I], q_pos [n_seq,n_q] i64, optional e_count [n_seq] i32. ``scores``
    is [n_seq, n_q, e_cap]: entries at or past a row's visible count are not written."""

    def __init__(self, q_idx, w, k_idx, q_pos, m: int, e_count=None):
        _dev(q_idx, "q_idx"); _dev(w, "w", torch.float32); _dev(k_idx, "k_idx", q_idx.dtype)
        _dev(q_pos, "q_pos", torch.int64); _dev(e_count, "e_count", torch.int32)
        self.args = (q_idx, w, k_idx, q_pos, e_count)
        n_seq, n_q, H, d = q_idx.shape
        e_cap = k_idx.shape[1]
        self.shape = (n_seq, n_q, e_cap, H, d, m)
        stride = (e_cap + 3) // 4 * 4
        self.rows = torch.empty(n_seq * n_q, stride, dtype=torch.float32, device=q_idx.device)
        self.scores = self.rows[:, :e_cap].view(n_seq, n_q, e_cap)
        nb = lib().csa_index_scores_workspace_size(n_seq, n_q, e_cap)
        self.ws = _workspace(nb, q_idx.device)

    def __call__(self):
        q_idx, w, k_idx, q_pos, e_count = self.args
        n_seq, n_q, e_cap, H, d, m = self.shape
        check("csa_index_scores", lib().csa_index_scores(
            _p(q_idx), _p(w), _p(k_idx), _p(q_pos), _p(e_count), n_seq, n_q, e_cap, H, d, m,
            _p(self.rows), self.rows.shape[1], _p(self.ws), self.ws.numel(), _dtype(q_idx),
            _stream()))
        return self.scores


def index_scores(q_idx, w, k_idx, q_pos, m: int, e_count=None):
    """csa_index_scores: every visible entry's index score, [n_seq, n_q, e_cap] f32 (entries at
    or past a row's visible count are not written)."""
    return IndexScores(q_idx, w, k_idx, q_pos, m, e_count)()


def index_blocks(q_idx, w, k_idx, q_pos, m: int, block_size: int, max_blocks: int,
                 e_count=None, top_k: int = 0):
    """csa_index_blocks: candidate pool [n_seq,n_q,max_blocks*block_size] (and the row's own
    Top-top_k when top_k > 0)."""
    _dev(q_idx, "q_idx"); _dev(w, "w", torch.float32); _dev(k_idx, "k_idx", q_idx.dtype)
    _dev(q_pos, "q_pos", torch.int64); _dev(e_count, "e_count", torch.int32)
    n_seq, n_q, H, d = q_idx.shape
    e_cap = k_idx.shape[1]
    dev = q_idx.device
    pool = torch.empty(n_seq, n_q, max_blocks * block_size, dtype=torch.int32, device=dev)
    out_idx = torch.empty(n_seq, n_q, top_k, dtype=torch.int32, device=dev) if top_k > 0 else None
    nb = lib().csa_index_blocks_workspace_size(n_seq, n_q, e_cap, block_size, max_blocks, top_k)
    ws = _workspace(nb, dev)
    check("csa_index_blocks", lib().csa_index_blocks(
        _p(q_idx), _p(w), _p(k_idx), _p(q_pos), _p(e_count), n_seq, n_q, e_cap, H, d, m,
        block_size, max_blocks, _p(pool), top_k, _p(out_idx), _p(ws), ws.numel(), _dtype(q_idx),
        _stream()))
    return pool if out_idx is None else (pool, out_idx)


def sparse_attn(q, kv, idx, win, w_cap: int, window: int, q_pos, sink, scale: float,
                out=None) -> torch.Tensor:
    """csa_sparse_attn. q [n_seq,n_q,H,D], kv [n_seq,e_cap,D], idx [n_seq,n_q,top_k] i32 or
    None, win [n_seq,w_cap,D] or None, q_pos [n_seq,n_q] i64, sink [H] f32 or None. A uint8 kv
    [n_seq,e_cap,576] is an FP8 main cache (quantize_kv_fp8's entries): csa_sparse_attn_fp8; a
    uint8 kv [n_seq,e_cap,288] an FP4 one (quantize_kv_fp4's entries): csa_sparse_attn_fp4."""
    fmt = _kv_entry_format(kv)
    kv8 = fmt != _lib.KV_DTYPE
    _dev(q, "q"); _dev(kv, "kv", torch.uint8 if kv8 else q.dtype); _dev(idx, "idx", torch.int32)
    _dev(win, "win", q.dtype); _dev(q_pos, "q_pos", torch.int64); _dev(sink, "sink", torch.float32)
    n_seq, n_q, H, D = q.shape
    e_cap = kv.shape[1]
    top_k = 0 if idx is None else idx.shape[-1]
    if out is None:
        out = torch.empty_like(q)
    nb = lib().csa_sparse_attn_workspace_size(n_seq, n_q, H, D, top_k, window)
    ws = _workspace(nb, q.device) if nb else None
    name = {_lib.KV_DTYPE: "csa_sparse_attn", _lib.KV_FP8: "csa_sparse_attn_fp8",
            _lib.KV_FP4: "csa_sparse_attn_fp4"}[fmt]
    check(name, getattr(lib(), name)(
        _p(q), _p(kv), _p(idx), top_k, _p(win), w_cap, window, _p(q_pos), _p(sink), float(scale),
        _p(out), n_seq, n_q, e_cap, H, D, _p(ws), 0 if ws is None else ws.numel(), _dtype(q),
        _stream()))
    return out


class DecodeStep:
    """csa_decode_step over caller-owned state. Builds the descriptor and its workspace once;
    each call runs one step (new token per sequence) on the current stream.

    Tensors (GPU, contiguous): pos, x_new, z_new, xi_new, zi_new, kv, k_idx, x_tail, z_tail,
    xi_tail, zi_tail, bias, bias_i, q_idx, w, [q_idx2, w2], q (list), win (list),
    win_new (list, entries may be None), sink (list, entries may be None); out (list) and
    out_idx are allocated here unless given. With k_idx_scale (uint8 [n_seq, e_cap,
    idx_dim / 32]) the indexer cache is MXFP4: k_idx holds the codes, uint8 [n_seq, e_cap,
    idx_dim / 2], as quantize_mxfp4 writes them; query_fp4=True then also takes the indexer
    query into MXFP4 (idx_format CSA_IDX_MXFP4_QK: the scan multiplies FP4 by FP4). score_format
    "bf16" ranks the index scores
    rounded to bf16. out_rope_dim > 0 applies the inverse RoPE (at -pos) to the last
    out_rope_dim channels of every output head, in the attention's output store. q_gamma (a
    list of [dim] tensors or None per call) and q_rope_dim prepare each call's query (RMSNorm,
    RoPE at +pos) in the selection launch. A uint8 kv [n_seq, e_cap, 576] is an FP8 main
    cache (quantize_kv_fp8's entries; kv_format CSA_KV_FP8), a uint8 kv [n_seq, e_cap, 288] an
    FP4 one (quantize_kv_fp4's entries; CSA_KV_FP4). kv_gamma ([dim] or None) and
    kv_rope_dim give the entry a step completes its RMSNorm and RoPE at pos before it is
    stored. compressor="c4a" pools the main entries with the overlapped two-stream compressor:
    x_new, z_new, x_tail, z_tail and bias are then its a stream, and xb_new, zb_new ([n_seq,
    dim]), xb_tail, zb_tail ([n_seq, 2m, dim], position p at row p % 2m) and bias_b ([m, dim])
    its b stream. With no_alloc=True no workspace is allocated and each call runs
    csa_decode_step_noalloc over the library's static per-GPU scratch array (calls that may
    overlap on one GPU race there)."""

    def __init__(self, *, m: int, top_k: int, window: int, scale: float, block_size: int = 0,
                 max_blocks: int = 0, out=None, out_idx=None, score_format: str = "f32",
                 out_rope_dim: int = 0, rope_base: float = 10000.0, q_gamma=None,
                 q_rope_dim: int = 0, kv_gamma=None, kv_rope_dim: int = 0,
                 compressor: str = "single", no_alloc: bool = False, query_fp4: bool = False,
                 **t):
        self.t = t
        kv = _dev(t["kv"], "kv")
        kv_fmt = _kv_entry_format(kv)
        kv8 = kv_fmt != _lib.KV_DTYPE
        dt = _dev(t["x_new"], "x_new").dtype if kv8 else kv.dtype
        mx = t.get("k_idx_scale") is not None
        for k in ("x_new", "z_new", "xi_new", "zi_new", "x_tail", "z_tail", "xi_tail",
                  "zi_tail", "bias", "bias_i", "q_idx"):
            _dev(t[k], k, dt)
        _dev(t["k_idx"], "k_idx", torch.uint8 if mx else dt)
        _dev(t["pos"], "pos", torch.int64)
        _dev(t["w"], "w", torch.float32)
        qs, wins = list(t["q"]), list(t["win"])
        n_attn = len(qs)
        win_new = list(t.get("win_new") or [])
        win_new += [None] * (n_attn - len(win_new))
        sinks = list(t.get("sink") or [])
        sinks += [None] * (n_attn - len(sinks))
        n_seq, e_cap, dim = kv.shape
        if kv8:
            dim = 512
        H = qs[0].shape[1]
        idx_heads, idx_dim = t["q_idx"].shape[1], t["q_idx"].shape[2]
        w_cap = wins[0].shape[1]
        if out is None:
            out = [torch.empty_like(q) for q in qs]
        if out_idx is None:
            out_idx = torch.empty(n_seq, top_k, dtype=torch.int32, device=kv.device)
        self.out, self.out_idx = out, out_idx
        d = DecodeDesc()
        d.dtype = _dtype(t["x_new"]); d.m = m; d.dim = dim; d.n_heads = H; d.idx_heads = idx_heads
        d.idx_dim = idx_dim; d.top_k = top_k; d.window = window; d.w_cap = w_cap
        d.block_size = block_size; d.max_blocks = max_blocks; d.n_attn = n_attn
        d.n_seq = n_seq; d.e_cap = e_cap; d.scale = float(scale)
        for k in ("pos", "x_new", "z_new", "xi_new", "zi_new", "kv", "k_idx", "x_tail", "z_tail",
                  "xi_tail", "zi_tail", "bias", "bias_i", "q_idx", "w"):
            setattr(d, k, t[k].data_ptr())
        if mx:
            ks = _dev(t["k_idx_scale"], "k_idx_scale", torch.uint8)
            if (tuple(t["k_idx"].shape) != (n_seq, e_cap, idx_dim // 2)
                    or tuple(ks.shape) != (n_seq, e_cap, idx_dim // 32)):
                raise ValueError("MXFP4 k_idx / k_idx_scale shapes do not match kv and q_idx")
            d.idx_format = _lib.IDX_MXFP4_QK if query_fp4 else _lib.IDX_MXFP4
            d.k_idx_scale = ks.data_ptr()
        elif query_fp4:
            raise ValueError("query_fp4 needs an MXFP4 indexer cache (k_idx_scale)")
        if block_size > 0:
            _dev(t["q_idx2"], "q_idx2", dt); _dev(t["w2"], "w2", torch.float32)
            d.q_idx2 = t["q_idx2"].data_ptr(); d.w2 = t["w2"].data_ptr()
        for c in range(n_attn):
            _dev(qs[c], "q", dt); _dev(wins[c], "win", dt); _dev(out[c], "out", dt)
            d.q[c] = qs[c].data_ptr(); d.win[c] = wins[c].data_ptr(); d.out[c] = out[c].data_ptr()
            if win_new[c] is not None:
                d.win_new[c] = _dev(win_new[c], "win_new", dt).data_ptr()
            if sinks[c] is not None:
                d.sink[c] = _dev(sinks[c], "sink", torch.float32).data_ptr()
        if score_format not in ("f32", "bf16"):
            raise ValueError("score_format must be 'f32' or 'bf16'")
        d.score_format = _lib.SCORE_BF16 if score_format == "bf16" else _lib.SCORE_F32
        d.out_rope_dim = int(out_rope_dim)
        d.rope_base = float(rope_base)
        d.q_rope_dim = int(q_rope_dim)
        self.q_gamma = list(q_gamma or [])   # the descriptor holds their addresses
        for c, gq in enumerate(self.q_gamma[:n_attn]):
            if gq is not None:
                d.q_gamma[c] = _dev(gq, "q_gamma", dt).data_ptr()
        d.kv_format = kv_fmt
        self.kv_gamma = kv_gamma   # the descriptor holds its address
        if kv_gamma is not None:
            d.kv_gamma = _dev(kv_gamma, "kv_gamma", dt).data_ptr()
        d.kv_rope_dim = int(kv_rope_dim)
        if compressor not in ("single", "c4a"):
            raise ValueError("compressor must be 'single' or 'c4a'")
        if compressor == "c4a":
            d.compressor = _lib.COMP_C4A
            want = {"xb_new": (n_seq, dim), "zb_new": (n_seq, dim), "xb_tail": (n_seq, 2 * m, dim),
                    "zb_tail": (n_seq, 2 * m, dim), "bias_b": (m, dim)}
            for k, shape in want.items():
                if tuple(_dev(t[k], k, dt).shape) != shape:
                    raise ValueError(f"{k} must be {list(shape)}")
                setattr(d, k, t[k].data_ptr())
        d.out_idx = out_idx.data_ptr()
        self.desc = d
        nb = lib().csa_decode_step_workspace_size(C.byref(d))
        if nb == 0:
            check("csa_decode_step_workspace_size", lib().csa_decode_step(C.byref(d), None, 0, None))
        self.no_alloc = no_alloc
        if no_alloc and nb > _lib.NOALLOC_SCRATCH_BYTES:
            raise ValueError(f"the step needs {nb} bytes of workspace, more than the "
                             f"{_lib.NOALLOC_SCRATCH_BYTES} of the static scratch")
        self.ws = None if no_alloc else _workspace(nb, kv.device)

    def set_events(self, handles) -> None:
        """Phase-boundary hipEvent_t handles (ints or None) recorded by the step."""
        hs = list(handles) + [None] * (_lib.DECODE_EVENTS - len(handles))
        for i, h in enumerate(hs[:_lib.DECODE_EVENTS]):
            self.desc.events[i] = h

    def set_scan_events(self, start=None, stop=None) -> None:
        """hipEvent_t handles (ints or None) taken by the indexer scan kernel's own dispatch."""
        if (start is None) != (stop is None):
            raise ValueError("set both scan events or neither")
        self.desc.scan_events[0] = start
        self.desc.scan_events[1] = stop

    def __call__(self, stream: int | None = None):
        s = _stream() if stream is None else stream
        if self.no_alloc:
            check("csa_decode_step_noalloc", lib().csa_decode_step_noalloc(C.byref(self.desc), s))
        else:
            check("csa_decode_step", lib().csa_decode_step(
                C.byref(self.desc), self.ws.data_ptr(), self.ws.numel(), s))
        return self.out, self.out_idx
