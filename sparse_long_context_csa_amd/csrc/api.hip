// C ABI of libcsa: argument validation (host, before any launch), workspace layout and the
// order of launches for each entry point. See include/csa.h for the contract.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "csa.h"
#include "launch.hpp"

using namespace csa;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }
int64_t round64(int64_t v) { return (v + 63) & ~int64_t(63); }

// Sequential sub-allocation of a caller workspace (sizes only when base == nullptr).
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T> T* take(size_t bytes) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += align_up(bytes);
    return p;
  }
};

bool dtype_ok(int32_t dt) { return dt == CSA_F32 || dt == CSA_BF16; }
int status_of(hipError_t e) { return e == hipSuccess ? CSA_OK : CSA_ERR_HIP; }

// ---- csa_index_topk workspace ------------------------------------------------------------
struct TopkWs {
  float* scores;
  uint32_t* gmax;     // order keys of the maxima of 16 consecutive scores (written by the scan)
  int32_t* n_vis;
  int32_t* count;
  void* scratch;
  void* seg;          // candidate segments of long decode rows (null when not carved)
  int64_t stride, gstride;
};
// few query rows per sequence: the scan is the decode kernel (as in launch_scan)
bool decode_rows(int64_t n_q) { return n_q < 16; }
TopkWs carve_topk(Carver& c, int64_t rows, int64_t n_keys, int32_t top_k, int64_t n_q) {
  TopkWs w;
  w.stride = round64(n_keys > 0 ? n_keys : 1);
  w.scores = c.take<float>(size_t(rows) * w.stride * 4);
  w.gstride = round64((n_keys > 0 ? n_keys : 1) / 16 + 1);
  w.gmax = c.take<uint32_t>(size_t(rows) * w.gstride * 4);
  w.n_vis = c.take<int32_t>(size_t(rows) * 4);
  w.count = c.take<int32_t>(size_t(rows) * 4);
  w.scratch = c.take<char>(topk_scratch_bytes(rows, n_keys, top_k));
  w.seg = nullptr;
  if (decode_rows(n_q) && n_keys > kSegRowMin) w.seg = c.take<char>(seg_bytes(rows, n_keys));
  return w;
}

// The scan's own workspace when its scores go to a caller buffer (csa_index_scores): visible
// counts and per-16-position maxima; no selection scratch, no segments.
TopkWs carve_scan_only(Carver& c, int64_t rows, int64_t n_keys) {
  TopkWs w{};
  w.gstride = round64(n_keys / 16 + 1);
  w.gmax = c.take<uint32_t>(size_t(rows) * w.gstride * 4);
  w.n_vis = c.take<int32_t>(size_t(rows) * 4);
  w.count = c.take<int32_t>(size_t(rows) * 4);
  return w;
}

// Segments of the decode scan for the select, when the scan is the bf16 64x128 decode kernel
// over the whole cache (no candidate list) and rows are long; both the scan and the select
// call this with the same arguments.
SegArgs segments_for(const TopkWs& ws, int dt, int H, int d, int64_t n_q, bool cand,
                     int64_t rows, int64_t n_keys, int K) {
  SegArgs g{};
  if (ws.seg == nullptr || cand || !decode_rows(n_q) || n_keys <= kSegRowMin) return g;
  if (!(dt == kBF16 && H == 64 && d == 128)) return g;
  return seg_carve(ws.seg, rows, n_keys, K);
}

// ---- csa_index_blocks workspace ----------------------------------------------------------
struct BlocksWs {
  TopkWs tk;          // stage-1 scores (+ scratch for the own Top-K)
  float* bmax;
  int32_t* nb;
  int32_t* blocks;
  void* scratch2;     // Top-K scratch for the block maxima
  int64_t bstride;
};
BlocksWs carve_blocks(Carver& c, int64_t rows, int64_t e_cap, int32_t bs, int32_t mb,
                      int32_t top_k, int64_t n_q) {
  BlocksWs w;
  w.tk = carve_topk(c, rows, e_cap, top_k > 0 ? top_k : 1, n_q);
  const int64_t nbmax = (e_cap + bs - 1) / bs;
  w.bstride = round64(nbmax);
  w.bmax = c.take<float>(size_t(rows) * w.bstride * 4);
  w.nb = c.take<int32_t>(size_t(rows) * 4);
  w.blocks = c.take<int32_t>(size_t(rows) * mb * 4);
  w.scratch2 = c.take<char>(topk_scratch_bytes(rows, nbmax, mb));
  return w;
}

int check_index_common(int64_t n_seq, int64_t n_q, int64_t e_cap, int32_t H, int32_t d,
                       int32_t m, int32_t dtype) {
  if (!dtype_ok(dtype)) return CSA_ERR_DTYPE;
  if (n_seq < 0 || n_q < 0 || e_cap < 1 || e_cap >= (int64_t(1) << 31)) return CSA_ERR_SHAPE;
  if (n_seq > 65535 || n_q * n_seq > 65535) return CSA_ERR_UNSUPPORTED;  // grid.y = rows
  if (H < 1 || H > 64 || d < 8 || d > 256 || (d % 8) != 0) return CSA_ERR_SHAPE;
  if (int64_t(H) * d > 8192) return CSA_ERR_UNSUPPORTED;
  if (m < 1 || m > 16) return CSA_ERR_SHAPE;
  return CSA_OK;
}

// scan of rows into a TopkWs (shared by the calls and the decode step)
hipError_t scan_rows(int dt, const void* q, const float* w, const void* keys, const int64_t* q_pos,
                     const int32_t* e_count, const int32_t* cand, int64_t n_cand, int64_t n_seq,
                     int64_t n_q, int64_t e_cap, int H, int d, int m, const TopkWs& ws,
                     hipStream_t s, const IngestArgs* ingest = nullptr, int seg_k = 0,
                     void* const* kernel_events = nullptr, const void* key_scales = nullptr,
                     bool score_bf16 = false, bool q_fp4 = false) {
  ScanArgs a{};
  a.dt = dt; a.q = q; a.w = w; a.keys = keys; a.q_pos = q_pos; a.e_count = e_count;
  a.key_scales = static_cast<const uint8_t*>(key_scales);
  a.score_bf16 = score_bf16 ? 1 : 0;
  a.q_fp4 = q_fp4 ? 1 : 0;
  a.cand = cand; a.n_cand = n_cand; a.n_seq = n_seq; a.n_q = n_q; a.e_cap = e_cap;
  a.H = H; a.d = d; a.m = m; a.scores = ws.scores; a.score_stride = ws.stride;
  a.n_vis = ws.n_vis; a.count = ws.count;
  a.gmax = ws.gmax; a.gmax_stride = ws.gstride;
  a.ingest = ingest ? *ingest : IngestArgs{};
  a.seg = seg_k > 0 ? segments_for(ws, dt, H, d, n_q, cand != nullptr, n_seq * n_q, e_cap, seg_k)
                    : SegArgs{};
  return launch_scan(a, s, kernel_events ? static_cast<hipEvent_t>(kernel_events[0]) : nullptr,
                     kernel_events ? static_cast<hipEvent_t>(kernel_events[1]) : nullptr);
}

hipError_t select_rows(const TopkWs& ws, int64_t rows, int64_t max_count, const int32_t* ids,
                       int64_t id_stride, const int32_t* id_limit, int K, int32_t* out_idx,
                       float* out_score, void* scratch, hipStream_t s,
                       const IngestArgs* side = nullptr, const SegArgs& seg = SegArgs{},
                       bool bf16_scores = false) {
  TopkArgs t{};
  t.scores = ws.scores; t.stride = ws.stride; t.ids = ids; t.id_stride = id_stride;
  t.gmax = ws.gmax; t.gstride = ws.gstride;
  t.id_limit = id_limit; t.count = ws.count; t.rows = rows; t.max_count = max_count; t.K = K;
  t.out_idx = out_idx; t.out_score = out_score; t.out_stride = K; t.scratch = scratch;
  t.side = side;
  t.seg = seg;
  t.bf16_scores = bf16_scores;
  return launch_topk(t, s);
}

// stage 1 of the hierarchical indexer after the scan: block maxima, top blocks, pool
hipError_t pool_rows(int64_t rows, int64_t e_cap, int bs, int mb, int32_t* out_pool,
                     const BlocksWs& ws, hipStream_t s) {
  hipError_t e = launch_block_max(ws.tk.scores, ws.tk.stride, ws.tk.count, rows, e_cap, bs,
                                  ws.bmax, ws.bstride, ws.nb, s);
  if (e != hipSuccess) return e;
  TopkArgs t{};
  t.scores = ws.bmax; t.stride = ws.bstride; t.ids = nullptr; t.id_stride = 0;
  t.gmax = nullptr; t.gstride = 0; t.side = nullptr;
  t.id_limit = nullptr; t.count = ws.nb; t.rows = rows; t.max_count = (e_cap + bs - 1) / bs;
  t.K = mb; t.out_idx = ws.blocks; t.out_score = nullptr; t.out_stride = mb;
  t.scratch = ws.scratch2;
  e = launch_topk(t, s);
  if (e != hipSuccess) return e;
  return launch_pool_build(ws.blocks, rows, mb, bs, ws.tk.n_vis, out_pool, s);
}

// stage 1 of the hierarchical indexer: scan, (own Top-K), block maxima, top blocks, pool
hipError_t blocks_rows(int dt, const void* q, const float* w, const void* keys,
                       const int64_t* q_pos, const int32_t* e_count, int64_t n_seq, int64_t n_q,
                       int64_t e_cap, int H, int d, int m, int bs, int mb, int32_t* out_pool,
                       int top_k, int32_t* out_idx, const BlocksWs& ws, hipStream_t s) {
  const int64_t rows = n_seq * n_q;
  hipError_t e = scan_rows(dt, q, w, keys, q_pos, e_count, nullptr, 0, n_seq, n_q, e_cap, H, d,
                           m, ws.tk, s, nullptr, out_idx ? top_k : 0);
  if (e != hipSuccess) return e;
  if (out_idx) {
    e = select_rows(ws.tk, rows, e_cap, nullptr, 0, nullptr, top_k, out_idx, nullptr,
                    ws.tk.scratch, s, nullptr,
                    segments_for(ws.tk, dt, H, d, n_q, false, rows, e_cap, top_k));
    if (e != hipSuccess) return e;
  }
  return pool_rows(rows, e_cap, bs, mb, out_pool, ws, s);
}

}  // namespace

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_status_str(int status) {
  switch (status) {
    case CSA_OK: return "ok";
    case CSA_ERR_NULL: return "a required pointer is NULL";
    case CSA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case CSA_ERR_DTYPE: return "unknown dtype";
    case CSA_ERR_UNSUPPORTED: return "request outside this build's limits";
    case CSA_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

// ---------------------------------------------------------------------------------------
int csa_compress(const void* x, const void* logits, const void* bias, void* out, int64_t n_seq,
                 int64_t n_tok, int64_t out_seq_stride, int32_t dim, int32_t m, int32_t dtype,
                 void* stream) {
  if (!dtype_ok(dtype)) return CSA_ERR_DTYPE;
  if (n_seq < 0 || n_tok < 0 || m < 1 || m > 128 || dim < 8 || dim > 8192 || (dim % 8) != 0)
    return CSA_ERR_SHAPE;
  if (n_tok % m != 0) return CSA_ERR_SHAPE;
  if (out_seq_stride != 0 && out_seq_stride < (n_tok / m) * dim) return CSA_ERR_SHAPE;
  if (out_seq_stride % 8 != 0) return CSA_ERR_SHAPE;
  if (n_seq * n_tok == 0) return CSA_OK;
  if (!x || !logits || !bias || !out) return CSA_ERR_NULL;
  return status_of(launch_compress(dtype, x, logits, bias, out, n_seq, n_tok, out_seq_stride,
                                   dim, m, static_cast<hipStream_t>(stream)));
}

int csa_compress_c4a(const void* xa, const void* za, const void* xb, const void* zb,
                     const void* bias_a, const void* bias_b, const void* xb_prev,
                     const void* zb_prev, void* out, int64_t n_seq, int64_t n_tok,
                     int64_t out_seq_stride, int32_t dim, int32_t m, int32_t dtype,
                     void* stream) {
  if (!dtype_ok(dtype)) return CSA_ERR_DTYPE;
  if (n_seq < 0 || n_tok < 0 || m < 1 || m > 16 || dim < 8 || dim > 8192 || (dim % 8) != 0)
    return CSA_ERR_SHAPE;
  if (n_tok % m != 0) return CSA_ERR_SHAPE;
  if (out_seq_stride != 0 && out_seq_stride < (n_tok / m) * dim) return CSA_ERR_SHAPE;
  if (out_seq_stride % 8 != 0) return CSA_ERR_SHAPE;
  if ((xb_prev == nullptr) != (zb_prev == nullptr)) return CSA_ERR_NULL;
  if (n_seq * n_tok == 0) return CSA_OK;
  if (!xa || !za || !xb || !zb || !bias_a || !bias_b || !out) return CSA_ERR_NULL;
  return status_of(launch_compress_c4a(dtype, xa, za, xb, zb, bias_a, bias_b, xb_prev, zb_prev,
                                       out, n_seq, n_tok, out_seq_stride, dim, m,
                                       static_cast<hipStream_t>(stream)));
}

int csa_norm_rope(const void* x, const void* gamma, const int64_t* pos, void* out,
                  int64_t n_rows, int32_t n_heads, int32_t dim, int32_t rope_dim,
                  float rope_base, float eps, int32_t flags, int32_t dtype, void* stream) {
  if (!dtype_ok(dtype)) return CSA_ERR_DTYPE;
  if (n_rows < 0 || n_heads < 1 || dim < 8 || dim > 512 || dim % 8 != 0) return CSA_ERR_SHAPE;
  if (rope_dim < 0 || rope_dim > dim || rope_dim % 2 != 0) return CSA_ERR_SHAPE;
  if (!(rope_base > 1.f) || !(eps >= 0.f) || (flags & ~7) != 0) return CSA_ERR_SHAPE;
  if ((flags & CSA_NR_INVERSE) && !(flags & CSA_NR_ROPE)) return CSA_ERR_SHAPE;
  if (n_rows == 0) return CSA_OK;
  if (!x || !out) return CSA_ERR_NULL;
  if ((flags & CSA_NR_NORM) && !gamma) return CSA_ERR_NULL;
  if ((flags & CSA_NR_ROPE) && !pos) return CSA_ERR_NULL;
  return status_of(launch_norm_rope(dtype, x, gamma, pos, out, n_rows, n_heads, dim, rope_dim,
                                    rope_base, eps, flags, static_cast<hipStream_t>(stream)));
}

int csa_quantize_mxfp4(const void* x, void* codes, void* scales, int64_t n_rows, int32_t dim,
                       int32_t dtype, void* stream) {
  if (!dtype_ok(dtype)) return CSA_ERR_DTYPE;
  if (n_rows < 0 || dim < 32 || dim > 8192 || dim % 32 != 0) return CSA_ERR_SHAPE;
  if (n_rows == 0) return CSA_OK;
  if (!x || !codes || !scales) return CSA_ERR_NULL;
  return status_of(launch_quantize_mxfp4(dtype, x, codes, scales, n_rows, dim,
                                         static_cast<hipStream_t>(stream)));
}

int csa_quantize_kv_fp8(const void* x, void* out, int64_t n_rows, int32_t dtype, void* stream) {
  if (!dtype_ok(dtype)) return CSA_ERR_DTYPE;
  if (n_rows < 0) return CSA_ERR_SHAPE;
  if (n_rows == 0) return CSA_OK;
  if (!x || !out) return CSA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(out) % 16 != 0) return CSA_ERR_SHAPE;
  return status_of(launch_quantize_kv_fp8(dtype, x, out, n_rows, static_cast<hipStream_t>(stream)));
}

int csa_dequantize_kv_fp8(const void* in, void* out, int64_t n_rows, void* stream) {
  if (n_rows < 0) return CSA_ERR_SHAPE;
  if (n_rows == 0) return CSA_OK;
  if (!in || !out) return CSA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(in) % 16 != 0 || reinterpret_cast<uintptr_t>(out) % 16 != 0)
    return CSA_ERR_SHAPE;
  return status_of(launch_dequantize_kv_fp8(in, out, n_rows, static_cast<hipStream_t>(stream)));
}

int csa_quantize_kv_fp4(const void* x, void* out, int64_t n_rows, int32_t dtype, void* stream) {
  if (!dtype_ok(dtype)) return CSA_ERR_DTYPE;
  if (n_rows < 0) return CSA_ERR_SHAPE;
  if (n_rows == 0) return CSA_OK;
  if (!x || !out) return CSA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(out) % 16 != 0) return CSA_ERR_SHAPE;
  return status_of(launch_quantize_kv_fp4(dtype, x, out, n_rows, static_cast<hipStream_t>(stream)));
}

int csa_dequantize_kv_fp4(const void* in, void* out, int64_t n_rows, void* stream) {
  if (n_rows < 0) return CSA_ERR_SHAPE;
  if (n_rows == 0) return CSA_OK;
  if (!in || !out) return CSA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(in) % 16 != 0 || reinterpret_cast<uintptr_t>(out) % 16 != 0)
    return CSA_ERR_SHAPE;
  return status_of(launch_dequantize_kv_fp4(in, out, n_rows, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------------------
size_t csa_index_topk_workspace_size(int64_t n_seq, int64_t n_q, int64_t n_keys, int32_t top_k) {
  if (n_seq < 0 || n_q < 0 || n_keys < 0 || top_k < 1) return 0;
  Carver c(nullptr);
  carve_topk(c, n_seq * n_q, n_keys, top_k, n_q);
  return c.off;
}

int csa_index_topk(const void* q_idx, const float* w, const void* k_idx, const int64_t* q_pos,
                   const int32_t* e_count, const int32_t* cand, int32_t n_cand, int64_t n_seq,
                   int64_t n_q, int64_t e_cap, int32_t idx_heads, int32_t idx_dim, int32_t m,
                   int32_t top_k, int32_t* out_idx, float* out_score, float* scores_all,
                   void* ws, size_t ws_bytes, int32_t dtype, void* stream) {
  int st = check_index_common(n_seq, n_q, e_cap, idx_heads, idx_dim, m, dtype);
  if (st != CSA_OK) return st;
  if (top_k < 1 || top_k > 2048) return CSA_ERR_SHAPE;
  if (n_cand < 0 || n_cand > 65536) return CSA_ERR_SHAPE;
  if (n_seq * n_q == 0) return CSA_OK;
  if (!q_idx || !w || !k_idx || !q_pos || !out_idx) return CSA_ERR_NULL;
  if (cand == nullptr && n_cand != 0) return CSA_ERR_NULL;
  const int64_t n_keys = cand ? n_cand : e_cap;
  const size_t need = csa_index_topk_workspace_size(n_seq, n_q, n_keys, top_k);
  if (!ws || ws_bytes < need) return CSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c(ws);
  const TopkWs tw = carve_topk(c, n_seq * n_q, n_keys, top_k, n_q);
  hipError_t e = scan_rows(dtype, q_idx, w, k_idx, q_pos, e_count, cand, n_cand, n_seq, n_q,
                           e_cap, idx_heads, idx_dim, m, tw, s, nullptr, top_k);
  if (e != hipSuccess) return CSA_ERR_HIP;
  e = select_rows(tw, n_seq * n_q, n_keys, cand, n_cand, cand ? tw.n_vis : nullptr, top_k,
                  out_idx, out_score, tw.scratch, s, nullptr,
                  segments_for(tw, dtype, idx_heads, idx_dim, n_q, cand != nullptr, n_seq * n_q,
                               n_keys, top_k));
  if (e != hipSuccess) return CSA_ERR_HIP;
  if (scores_all) {
    e = launch_fill_scores(tw.scores, tw.stride, tw.count, n_seq * n_q, n_keys, scores_all, s);
    if (e != hipSuccess) return CSA_ERR_HIP;
  }
  return CSA_OK;
}

// ---------------------------------------------------------------------------------------
size_t csa_index_scores_workspace_size(int64_t n_seq, int64_t n_q, int64_t e_cap) {
  if (n_seq < 0 || n_q < 0 || e_cap < 1) return 0;
  Carver c(nullptr);
  carve_scan_only(c, n_seq * n_q, e_cap);
  return c.off;
}

int csa_index_scores(const void* q_idx, const float* w, const void* k_idx, const int64_t* q_pos,
                     const int32_t* e_count, int64_t n_seq, int64_t n_q, int64_t e_cap,
                     int32_t idx_heads, int32_t idx_dim, int32_t m, float* scores,
                     int64_t score_stride, void* ws, size_t ws_bytes, int32_t dtype,
                     void* stream) {
  int st = check_index_common(n_seq, n_q, e_cap, idx_heads, idx_dim, m, dtype);
  if (st != CSA_OK) return st;
  if (score_stride < e_cap || score_stride % 4 != 0) return CSA_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(scores) % 16 != 0) return CSA_ERR_SHAPE;
  if (n_seq * n_q == 0) return CSA_OK;
  if (!q_idx || !w || !k_idx || !q_pos || !scores) return CSA_ERR_NULL;
  const size_t need = csa_index_scores_workspace_size(n_seq, n_q, e_cap);
  if (!ws || ws_bytes < need) return CSA_ERR_WORKSPACE;
  Carver c(ws);
  TopkWs tw = carve_scan_only(c, n_seq * n_q, e_cap);
  tw.scores = scores;
  tw.stride = score_stride;
  return status_of(scan_rows(dtype, q_idx, w, k_idx, q_pos, e_count, nullptr, 0, n_seq, n_q,
                             e_cap, idx_heads, idx_dim, m, tw, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------------------
size_t csa_index_blocks_workspace_size(int64_t n_seq, int64_t n_q, int64_t e_cap,
                                       int32_t block_size, int32_t max_blocks, int32_t top_k) {
  if (n_seq < 0 || n_q < 0 || e_cap < 1 || block_size < 1 || max_blocks < 1) return 0;
  Carver c(nullptr);
  carve_blocks(c, n_seq * n_q, e_cap, block_size, max_blocks, top_k, n_q);
  return c.off;
}

int csa_index_blocks(const void* q_idx, const float* w, const void* k_idx, const int64_t* q_pos,
                     const int32_t* e_count, int64_t n_seq, int64_t n_q, int64_t e_cap,
                     int32_t idx_heads, int32_t idx_dim, int32_t m, int32_t block_size,
                     int32_t max_blocks, int32_t* out_pool, int32_t top_k, int32_t* out_idx,
                     void* ws, size_t ws_bytes, int32_t dtype, void* stream) {
  int st = check_index_common(n_seq, n_q, e_cap, idx_heads, idx_dim, m, dtype);
  if (st != CSA_OK) return st;
  if (block_size < 1 || block_size > 64 || max_blocks < 1) return CSA_ERR_SHAPE;
  if (int64_t(block_size) * max_blocks > 32768) return CSA_ERR_UNSUPPORTED;
  if (out_idx && (top_k < 1 || top_k > 2048)) return CSA_ERR_SHAPE;
  if (max_blocks > 2048) return CSA_ERR_UNSUPPORTED;
  if (n_seq * n_q == 0) return CSA_OK;
  if (!q_idx || !w || !k_idx || !q_pos || !out_pool) return CSA_ERR_NULL;
  const int32_t tk = out_idx ? top_k : 0;
  const size_t need = csa_index_blocks_workspace_size(n_seq, n_q, e_cap, block_size, max_blocks, tk);
  if (!ws || ws_bytes < need) return CSA_ERR_WORKSPACE;
  Carver c(ws);
  const BlocksWs bw = carve_blocks(c, n_seq * n_q, e_cap, block_size, max_blocks, tk, n_q);
  return status_of(blocks_rows(dtype, q_idx, w, k_idx, q_pos, e_count, n_seq, n_q, e_cap,
                               idx_heads, idx_dim, m, block_size, max_blocks, out_pool, tk,
                               out_idx, bw, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------------------
size_t csa_sparse_attn_workspace_size(int64_t n_seq, int64_t n_q, int32_t n_heads,
                                      int32_t head_dim, int32_t top_k, int32_t window) {
  if (n_seq < 0 || n_q < 0 || top_k < 0 || window < 0) return 0;
  // the split plan depends on the dtype only through the fast-path test; size for bf16
  return align_up(attn_ws_bytes(n_seq * n_q, n_heads, head_dim, top_k, window, CSA_BF16));
}

static int check_attn(int64_t n_seq, int64_t n_q, int64_t e_cap, int32_t H, int32_t D,
                      int32_t top_k, int32_t w_cap, int32_t window, int32_t dtype) {
  if (!dtype_ok(dtype)) return CSA_ERR_DTYPE;
  if (n_seq < 0 || n_q < 0 || e_cap < 1 || e_cap >= (int64_t(1) << 31)) return CSA_ERR_SHAPE;
  if (n_seq > 65535 || n_seq * n_q > 65535) return CSA_ERR_UNSUPPORTED;  // grid.y = rows
  if (H < 1 || H > 64 || D < 8 || D > 512 || (D % 8) != 0) return CSA_ERR_SHAPE;
  if (top_k < 0 || top_k > 16384 || window < 0) return CSA_ERR_SHAPE;
  if (window > 0 && (w_cap < 1 || window > w_cap)) return CSA_ERR_SHAPE;
  return CSA_OK;
}

static int sparse_attn_impl(const void* q, const void* kv, const int32_t* idx, int32_t top_k,
                            const void* win, int32_t w_cap, int32_t window,
                            const int64_t* q_pos, const float* sink, float scale, void* out,
                            int64_t n_seq, int64_t n_q, int64_t e_cap, int32_t n_heads,
                            int32_t head_dim, void* ws, size_t ws_bytes, int32_t dtype,
                            int kv_fmt, void* stream) {
  int st = check_attn(n_seq, n_q, e_cap, n_heads, head_dim, top_k, w_cap, window, dtype);
  if (st != CSA_OK) return st;
  if (kv_fmt != kKvPlain) {
    if (dtype != CSA_BF16 || n_heads != 64 || head_dim != 512) return CSA_ERR_UNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(kv) % 16 != 0) return CSA_ERR_SHAPE;
  }
  if (n_seq * n_q == 0) return CSA_OK;
  if (!q || !q_pos || !out) return CSA_ERR_NULL;
  if (top_k > 0 && (!idx || !kv)) return CSA_ERR_NULL;
  if (window > 0 && !win) return CSA_ERR_NULL;
  const size_t need = csa_sparse_attn_workspace_size(n_seq, n_q, n_heads, head_dim, top_k, window);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  AttnArgs a{};
  a.dt = dtype; a.q = q; a.kv = kv; a.idx = idx; a.top_k = top_k; a.win = win; a.w_cap = w_cap;
  a.window = window; a.q_pos = q_pos; a.sink = sink; a.scale = scale; a.out = out;
  a.n_seq = n_seq; a.n_q = n_q; a.e_cap = e_cap; a.H = n_heads; a.D = head_dim; a.ws = ws;
  a.kv_fmt = kv_fmt;
  return status_of(launch_attn(a, static_cast<hipStream_t>(stream)));
}

int csa_sparse_attn(const void* q, const void* kv, const int32_t* idx, int32_t top_k,
                    const void* win, int32_t w_cap, int32_t window, const int64_t* q_pos,
                    const float* sink, float scale, void* out, int64_t n_seq, int64_t n_q,
                    int64_t e_cap, int32_t n_heads, int32_t head_dim, void* ws, size_t ws_bytes,
                    int32_t dtype, void* stream) {
  return sparse_attn_impl(q, kv, idx, top_k, win, w_cap, window, q_pos, sink, scale, out, n_seq,
                          n_q, e_cap, n_heads, head_dim, ws, ws_bytes, dtype, kKvPlain, stream);
}

int csa_sparse_attn_fp8(const void* q, const void* kv, const int32_t* idx, int32_t top_k,
                        const void* win, int32_t w_cap, int32_t window, const int64_t* q_pos,
                        const float* sink, float scale, void* out, int64_t n_seq, int64_t n_q,
                        int64_t e_cap, int32_t n_heads, int32_t head_dim, void* ws,
                        size_t ws_bytes, int32_t dtype, void* stream) {
  return sparse_attn_impl(q, kv, idx, top_k, win, w_cap, window, q_pos, sink, scale, out, n_seq,
                          n_q, e_cap, n_heads, head_dim, ws, ws_bytes, dtype, kKvFp8, stream);
}

int csa_sparse_attn_fp4(const void* q, const void* kv, const int32_t* idx, int32_t top_k,
                        const void* win, int32_t w_cap, int32_t window, const int64_t* q_pos,
                        const float* sink, float scale, void* out, int64_t n_seq, int64_t n_q,
                        int64_t e_cap, int32_t n_heads, int32_t head_dim, void* ws,
                        size_t ws_bytes, int32_t dtype, void* stream) {
  return sparse_attn_impl(q, kv, idx, top_k, win, w_cap, window, q_pos, sink, scale, out, n_seq,
                          n_q, e_cap, n_heads, head_dim, ws, ws_bytes, dtype, kKvFp4, stream);
}

// ---------------------------------------------------------------------------------------
namespace {
struct DecodeWs {
  TopkWs flat;        // flat: scan + select; hierarchical: stage-2 scores over the pool
  BlocksWs blocks;    // hierarchical stage 1
  int32_t* pool;
  void* attn;
  char* qprep;        // prepared queries [n_attn][n_seq, n_heads, dim] (when asked for)
};

bool wants_qprep(const csa_decode_desc* d) {
  if (d->q_rope_dim > 0) return true;
  for (int c = 0; c < d->n_attn && c < CSA_MAX_ATTN; ++c)
    if (d->q_gamma[c] != nullptr) return true;
  return false;
}
size_t q_bytes(const csa_decode_desc* d) {
  return size_t(d->n_seq) * d->n_heads * d->dim * (d->dtype == CSA_BF16 ? 2 : 4);
}
DecodeWs carve_decode(Carver& c, const csa_decode_desc* d) {
  DecodeWs w{};
  const int64_t rows = d->n_seq;
  if (d->block_size > 0) {
    const int64_t np = int64_t(d->block_size) * d->max_blocks;
    w.blocks = carve_blocks(c, rows, d->e_cap, d->block_size, d->max_blocks, 0, 1);
    w.pool = c.take<int32_t>(size_t(rows) * np * 4);
    w.flat = carve_topk(c, rows, np, d->top_k, 1);
  } else {
    w.flat = carve_topk(c, rows, d->e_cap, d->top_k, 1);
  }
  w.attn = c.take<char>(attn_ws_bytes(rows, d->n_heads, d->dim, d->top_k, d->window, CSA_BF16));
  if (wants_qprep(d)) w.qprep = c.take<char>(q_bytes(d) * size_t(d->n_attn));
  return w;
}

int kv_fmt_of(const csa_decode_desc* d) {
  return d->kv_format == CSA_KV_FP8 ? kKvFp8 : d->kv_format == CSA_KV_FP4 ? kKvFp4 : kKvPlain;
}

int check_decode_shapes(const csa_decode_desc* d) {
  if (!d) return CSA_ERR_NULL;
  if (!dtype_ok(d->dtype)) return CSA_ERR_DTYPE;
  if (d->n_seq < 0 || d->n_seq > 65535) return CSA_ERR_SHAPE;
  int st = check_index_common(d->n_seq, 1, d->e_cap, d->idx_heads, d->idx_dim, d->m, d->dtype);
  if (st != CSA_OK) return st;
  st = check_attn(d->n_seq, 1, d->e_cap, d->n_heads, d->dim, d->top_k, d->w_cap, d->window,
                  d->dtype);
  if (st != CSA_OK) return st;
  if (d->top_k < 1 || d->top_k > 2048) return CSA_ERR_SHAPE;
  if (d->n_attn < 1 || d->n_attn > CSA_MAX_ATTN) return CSA_ERR_SHAPE;
  if (d->block_size < 0) return CSA_ERR_SHAPE;
  if ((d->scan_events[0] == nullptr) != (d->scan_events[1] == nullptr)) return CSA_ERR_NULL;
  if (d->block_size > 0) {
    if (d->block_size > 64 || d->max_blocks < 1 || d->max_blocks > 2048) return CSA_ERR_SHAPE;
    if (int64_t(d->block_size) * d->max_blocks > 32768) return CSA_ERR_UNSUPPORTED;
  }
  if (d->idx_format != CSA_IDX_DTYPE && d->idx_format != CSA_IDX_MXFP4 &&
      d->idx_format != CSA_IDX_MXFP4_QK)
    return CSA_ERR_SHAPE;
  if (d->idx_format != CSA_IDX_DTYPE &&
      (d->block_size != 0 || !scan_fuses_ingest(d->dtype, d->idx_heads, d->idx_dim, d->m) ||
       !scan_reads_mxfp4(d->dtype, d->idx_heads, d->idx_dim, 1, false)))
    return CSA_ERR_UNSUPPORTED;
  if (d->out_rope_dim < 0 || d->out_rope_dim > d->dim || d->out_rope_dim % 2 != 0)
    return CSA_ERR_SHAPE;
  if (d->q_rope_dim < 0 || d->q_rope_dim > d->dim || d->q_rope_dim % 2 != 0)
    return CSA_ERR_SHAPE;
  if (d->q_rope_dim > 0 && !(d->rope_base > 1.f)) return CSA_ERR_SHAPE;
  if (d->q_rope_dim > 64) return CSA_ERR_UNSUPPORTED;   // 32 pair angles per row at most
  if (wants_qprep(d) && d->dim > 512) return CSA_ERR_UNSUPPORTED;
  if (d->out_rope_dim > 0) {
    if (!(d->rope_base > 1.f)) return CSA_ERR_SHAPE;
    if (d->dtype == CSA_BF16 && d->n_heads == 64 && d->dim == 512 && d->out_rope_dim % 16 != 0)
      return CSA_ERR_UNSUPPORTED;
  }
  if (d->kv_rope_dim < 0 || d->kv_rope_dim % 2 != 0 || d->kv_rope_dim > d->dim)
    return CSA_ERR_SHAPE;
  if (d->kv_rope_dim > 0 && !(d->rope_base > 1.f)) return CSA_ERR_SHAPE;
  if ((d->kv_gamma != nullptr || d->kv_rope_dim > 0) && (d->dim != 512 || d->kv_rope_dim > 64))
    return CSA_ERR_UNSUPPORTED;
  if (d->kv_format != CSA_KV_DTYPE && d->kv_format != CSA_KV_FP8 && d->kv_format != CSA_KV_FP4)
    return CSA_ERR_SHAPE;
  if (d->kv_format != CSA_KV_DTYPE && (d->dtype != CSA_BF16 || d->n_heads != 64 || d->dim != 512))
    return CSA_ERR_UNSUPPORTED;
  if (d->score_format != CSA_SCORE_F32 && d->score_format != CSA_SCORE_BF16) return CSA_ERR_SHAPE;
  if (d->compressor != CSA_COMP_SINGLE && d->compressor != CSA_COMP_C4A) return CSA_ERR_SHAPE;
  if (d->score_format == CSA_SCORE_BF16 &&
      (d->block_size != 0 || !scan_reads_mxfp4(d->dtype, d->idx_heads, d->idx_dim, 1, false)))
    return CSA_ERR_UNSUPPORTED;
  return CSA_OK;
}

int check_decode(const csa_decode_desc* d) {
  int st = check_decode_shapes(d);
  if (st != CSA_OK) return st;
  if (d->n_seq == 0) return CSA_OK;
  if (!d->pos || !d->x_new || !d->z_new || !d->xi_new || !d->zi_new || !d->kv || !d->k_idx ||
      !d->x_tail || !d->z_tail || !d->xi_tail || !d->zi_tail || !d->bias || !d->bias_i ||
      !d->q_idx || !d->w || !d->out_idx)
    return CSA_ERR_NULL;
  if (d->block_size > 0 && (!d->q_idx2 || !d->w2)) return CSA_ERR_NULL;
  if (d->compressor == CSA_COMP_C4A &&
      (!d->xb_new || !d->zb_new || !d->xb_tail || !d->zb_tail || !d->bias_b))
    return CSA_ERR_NULL;
  if (d->idx_format != CSA_IDX_DTYPE) {
    if (!d->k_idx_scale) return CSA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(d->k_idx) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(d->k_idx_scale) % 4 != 0)
      return CSA_ERR_SHAPE;
  }
  if (d->kv_format != CSA_KV_DTYPE && reinterpret_cast<uintptr_t>(d->kv) % 16 != 0)
    return CSA_ERR_SHAPE;
  for (int c = 0; c < d->n_attn; ++c) {
    if (!d->q[c] || !d->out[c]) return CSA_ERR_NULL;
    if (d->window > 0 && !d->win[c]) return CSA_ERR_NULL;
    if (d->win_new[c] && !d->win[c]) return CSA_ERR_NULL;
  }
  return CSA_OK;
}
}  // namespace

size_t csa_decode_step_workspace_size(const csa_decode_desc* d) {
  if (check_decode_shapes(d) != CSA_OK) return 0;
  Carver c(nullptr);
  carve_decode(c, d);
  return c.off;
}

namespace {
// The decode step over a validated descriptor and a workspace of at least the bytes
// csa_decode_step_workspace_size gives (no kernel needs it cleared).
int decode_step_run(const csa_decode_desc* d, void* ws, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c(ws);
  const DecodeWs w = carve_decode(c, d);
  const int64_t rows = d->n_seq;
  auto mark = [&](int i) {
    if (d->events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(d->events[i]), s);
  };
  mark(0);

  // 1-2. new rows into tails / rings; pool the block when it completes
  IngestArgs in{};
  in.dt = d->dtype; in.n_seq = d->n_seq; in.e_cap = d->e_cap; in.m = d->m; in.dim = d->dim;
  in.idx_dim = d->idx_dim; in.w_cap = d->w_cap; in.n_ring = d->n_attn; in.pos = d->pos;
  in.x_new = d->x_new; in.z_new = d->z_new; in.xi_new = d->xi_new; in.zi_new = d->zi_new;
  in.x_tail = d->x_tail; in.z_tail = d->z_tail; in.xi_tail = d->xi_tail; in.zi_tail = d->zi_tail;
  in.bias = d->bias; in.bias_i = d->bias_i; in.kv = d->kv; in.k_idx = d->k_idx;
  void* key_scales = d->idx_format != CSA_IDX_DTYPE ? d->k_idx_scale : nullptr;
  in.k_scale = key_scales;
  in.kv_fmt = kv_fmt_of(d);
  in.kv_gamma = d->kv_gamma;
  in.kv_rope_dim = d->kv_rope_dim;
  if (d->compressor == CSA_COMP_C4A) {
    in.xb_new = d->xb_new; in.zb_new = d->zb_new; in.xb_tail = d->xb_tail;
    in.zb_tail = d->zb_tail; in.bias_b = d->bias_b;
  }
  in.rope_log2_base = d->rope_base > 1.f ? log2(double(d->rope_base)) : 0.0;
  for (int c2 = 0; c2 < 4; ++c2) {
    in.win[c2] = c2 < d->n_attn ? d->win[c2] : nullptr;
    in.win_new[c2] = (c2 < d->n_attn && d->w_cap > 0) ? d->win_new[c2] : nullptr;
  }
  // Where the decode scan can take it, the ingest is split between the stage-1 scan (the
  // completed entry's indexer key, which that scan scores) and extra workgroups of the last
  // select launch (tails, rings, main entry: read only by the attention). Otherwise it runs
  // first as a kernel of its own. Event 1 then marks the end of that kernel (or event 0).
  // the attention calls' queries, prepared by the ingest workgroups of the select launch (or
  // by one csa_norm_rope pass each when the ingest runs as a kernel of its own)
  if (w.qprep) {
    in.n_qprep = d->n_attn; in.q_heads = d->n_heads; in.q_dim = d->dim;
    in.q_rope_dim = d->q_rope_dim;
    for (int c2 = 0; c2 < d->n_attn; ++c2) {
      in.qsrc[c2] = d->q[c2];
      in.qgamma[c2] = d->q_gamma[c2];
      in.qdst[c2] = w.qprep + size_t(c2) * q_bytes(d);
    }
  }
  const bool fuse = scan_fuses_ingest(d->dtype, d->idx_heads, d->idx_dim, d->m);
  if (!fuse && launch_ingest(in, s) != hipSuccess) return CSA_ERR_HIP;
  if (!fuse && w.qprep) {
    for (int c2 = 0; c2 < d->n_attn; ++c2) {
      const int flags = (d->q_gamma[c2] ? CSA_NR_NORM : 0) | (d->q_rope_dim > 0 ? CSA_NR_ROPE : 0);
      if (flags != 0 &&
          launch_norm_rope(d->dtype, d->q[c2], d->q_gamma[c2], d->pos, in.qdst[c2], d->n_seq,
                           d->n_heads, d->dim, d->q_rope_dim, d->rope_base, 1e-6f, flags, s) !=
              hipSuccess)
        return CSA_ERR_HIP;
    }
  }
  const IngestArgs* split_ingest = fuse ? &in : nullptr;
  mark(1);

  // 3-4. index + select
  if (d->block_size > 0) {
    const int np = d->block_size * d->max_blocks;
    if (scan_rows(d->dtype, d->q_idx, d->w, d->k_idx, d->pos, nullptr, nullptr, 0, rows, 1,
                  d->e_cap, d->idx_heads, d->idx_dim, d->m, w.blocks.tk, s, split_ingest, 0,
                  d->scan_events) != hipSuccess)
      return CSA_ERR_HIP;
    mark(2);
    if (pool_rows(rows, d->e_cap, d->block_size, d->max_blocks, w.pool, w.blocks, s) != hipSuccess)
      return CSA_ERR_HIP;
    if (scan_rows(d->dtype, d->q_idx2, d->w2, d->k_idx, d->pos, nullptr, w.pool, np, rows, 1,
                  d->e_cap, d->idx_heads, d->idx_dim, d->m, w.flat, s) != hipSuccess)
      return CSA_ERR_HIP;
    if (select_rows(w.flat, rows, np, w.pool, np, w.flat.n_vis, d->top_k, d->out_idx, nullptr,
                    w.flat.scratch, s, split_ingest) != hipSuccess)
      return CSA_ERR_HIP;
  } else {
    if (scan_rows(d->dtype, d->q_idx, d->w, d->k_idx, d->pos, nullptr, nullptr, 0, rows, 1,
                  d->e_cap, d->idx_heads, d->idx_dim, d->m, w.flat, s, split_ingest,
                  d->top_k, d->scan_events, key_scales,
                  d->score_format == CSA_SCORE_BF16,
                  d->idx_format == CSA_IDX_MXFP4_QK) != hipSuccess)
      return CSA_ERR_HIP;
    mark(2);
    const SegArgs seg = segments_for(w.flat, d->dtype, d->idx_heads, d->idx_dim, 1, false, rows,
                                     d->e_cap, d->top_k);
    if (select_rows(w.flat, rows, d->e_cap, nullptr, 0, nullptr, d->top_k, d->out_idx, nullptr,
                    w.flat.scratch, s, split_ingest, seg,
                    d->score_format == CSA_SCORE_BF16) != hipSuccess)
      return CSA_ERR_HIP;
  }

  mark(3);
  // 5. attention calls sharing the selection, one after another
  for (int c2 = 0; c2 < d->n_attn; ++c2) {
    AttnArgs a{};
    a.dt = d->dtype; a.q = d->q[c2]; a.kv = d->kv; a.idx = d->out_idx; a.top_k = d->top_k;
    a.win = d->win[c2]; a.w_cap = d->w_cap; a.window = d->window; a.q_pos = d->pos;
    a.sink = d->sink[c2]; a.scale = d->scale; a.out = d->out[c2]; a.n_seq = d->n_seq;
    a.n_q = 1; a.e_cap = d->e_cap; a.H = d->n_heads; a.D = d->dim; a.ws = w.attn;
    a.out_rope_dim = d->out_rope_dim;
    a.kv_fmt = kv_fmt_of(d);
    if (w.qprep && (d->q_gamma[c2] != nullptr || d->q_rope_dim > 0))
      a.q = w.qprep + size_t(c2) * q_bytes(d);   // this call's prepared query
    a.rope_log2_base = d->out_rope_dim > 0 ? log2(double(d->rope_base)) : 0.0;
    if (launch_attn(a, s) != hipSuccess) return CSA_ERR_HIP;
  }
  mark(4);
  return CSA_OK;
}
}  // namespace

int csa_decode_step(const csa_decode_desc* d, void* ws, size_t ws_bytes, void* stream) {
  int st = check_decode(d);
  if (st != CSA_OK) return st;
  if (d->n_seq == 0) return CSA_OK;
  const size_t need = csa_decode_step_workspace_size(d);
  if (!ws || ws_bytes < need) return CSA_ERR_WORKSPACE;
  return decode_step_run(d, ws, stream);
}

}  // extern "C"

// ---- the allocation-free decode step ---------------------------------------------------
// The workspace lives in a file-scope device array. In host code `scratch` names a host-side
// stand-in, not the device memory: its device address on each GPU comes from
// hipGetSymbolAddress (every GPU the library runs on holds its own copy, at its own address,
// until the process ends) and only that address is ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[CSA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];   // per device: &scratch on that device, once found

// The device address of `scratch` on device `dev`, looked up once per device with that device
// current (the calling thread's current device is restored afterwards).
int scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxScratchDevices) return CSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return CSA_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return CSA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return CSA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSA_OK;
}
}  // namespace

extern "C" int csa_decode_step_noalloc(const csa_decode_desc* d, void* stream) {
  int st = check_decode(d);
  if (st != CSA_OK) return st;
  if (d->n_seq == 0) return CSA_OK;
  if (csa_decode_step_workspace_size(d) > CSA_NOALLOC_SCRATCH_BYTES) return CSA_ERR_WORKSPACE;
  int dev = -1;
  if (stream != nullptr) {
    hipDevice_t sd = 0;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sd) != hipSuccess)
      return CSA_ERR_HIP;
    dev = static_cast<int>(sd);
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return CSA_ERR_HIP;
  }
  void* ws = nullptr;
  st = scratch_address(dev, &ws);
  if (st != CSA_OK) return st;
  return decode_step_run(d, ws, stream);
}
