// Host-side launchers of the libcsa kernels (internal; the public ABI is include/csa.h).
// Every launcher enqueues on `stream` and returns hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

enum DType : int { kF32 = 0, kBF16 = 1 };
// kv_fmt of the attention and ingest arguments: how the main cache holds its entries
constexpr int kKvPlain = 0;   // the step's dtype, dim channels
constexpr int kKvFp8 = 1;     // 576-byte FP8 entries
constexpr int kKvFp4 = 2;     // 288-byte FP4 entries

// ---- compressor --------------------------------------------------------------------------
hipError_t launch_compress(int dt, const void* x, const void* z, const void* bias, void* out,
                           int64_t n_seq, int64_t n_tok, int64_t out_seq_stride, int dim, int m,
                           hipStream_t s);

// overlapped two-stream compressor: entry e pools a-rows [m e, m e + m) and b-rows
// [m(e-1), m e) (xb_prev/zb_prev [n_seq, m, dim] for e = 0, or none when null)
hipError_t launch_compress_c4a(int dt, const void* xa, const void* za, const void* xb,
                               const void* zb, const void* ba, const void* bb,
                               const void* xb_prev, const void* zb_prev, void* out,
                               int64_t n_seq, int64_t n_tok, int64_t out_seq_stride, int dim,
                               int m, hipStream_t s);

struct IngestArgs {
  int dt;
  int64_t n_seq, e_cap;
  int m, dim, idx_dim, w_cap, n_ring;
  const int64_t* pos;
  const void *x_new, *z_new, *xi_new, *zi_new;
  void *x_tail, *z_tail, *xi_tail, *zi_tail;
  const void *bias, *bias_i;
  void *kv, *k_idx;
  int kv_fmt;             // kKvPlain, kKvFp8 (576-byte entries) or kKvFp4 (288-byte entries)
  // the entry a step completes gets the per-head RMSNorm (kv_gamma [dim], or none when null)
  // and RoPE at t on its last kv_rope_dim channels before it is stored (dim == 512: the
  // entry's 64 vectors are the 64 lanes of one wave)
  const void* kv_gamma;
  int kv_rope_dim;
  void* k_scale;          // non-null: k_idx holds MXFP4 codes, k_scale their scale bytes
  // overlapped two-stream main compressor (xb_new non-null): the b stream's new row enters
  // xb_tail / zb_tail [n_seq, 2m, dim] at row t % 2m (position p at row p % 2m) and entry e
  // pools the a tail with the b rows of block e - 1, bias_b [m, dim] on the b logits
  const void *xb_new, *zb_new;
  void *xb_tail, *zb_tail;
  const void* bias_b;
  void* win[4];
  const void* win_new[4];
  // query preparation for the attention calls, done by the workgroups that run this ingest:
  // call c's query qsrc[c] [n_seq, q_heads, q_dim] gets the per-head RMSNorm (qgamma[c], or
  // none when null) and RoPE at +pos on its last q_rope_dim channels, into qdst[c]
  int n_qprep, q_heads, q_dim, q_rope_dim;
  double rope_log2_base;
  const void* qsrc[4];
  const void* qgamma[4];
  void* qdst[4];
};
hipError_t launch_ingest(const IngestArgs& a, hipStream_t s);

// ---- candidate segments of long decode rows -----------------------------------------------
// The decode scan cuts each row into chunks of positions (its work items). For rows longer
// than kSegRowMin it can also leave, per chunk c, the positions whose score key reaches a
// threshold tau_c of its own (the J-th largest of the chunk's 16-position maxima), in
// position order: seg[c][0 .. min(n_c, kChunkSegCap)), n_c in seg_n[c], (tau_c, the chunk's
// largest key) in seg_info[c]. The select then works on the segments alone and checks that
// every tau_c lies at or below the K-th key it finds (see topk.hip).
constexpr int64_t kSegRowMin = 32768;
constexpr int kChunkSegCap = 128;
constexpr int kSegMaxChunk = 2048;
struct SegArgs {
  uint2* seg;             // [rows][nseg][kChunkSegCap] (key, position); null: no segments
  int32_t* seg_n;         // [rows][nseg]
  uint2* seg_info;        // [rows][nseg]
  int64_t nseg;           // chunks per row (row stride of the arrays)
  int chunk;              // positions per chunk
  int K;
};
// Positions per decode-scan work item for `rows` rows of up to `max_pos` positions (segment
// chunks when segments are written), and the buffer sizes of the segments.
int decode_scan_chunk(int64_t rows, int64_t max_pos, bool segments);
size_t seg_bytes(int64_t rows, int64_t max_pos);
// carves the three arrays out of `base` (seg_bytes long); sets nseg and chunk
SegArgs seg_carve(void* base, int64_t rows, int64_t max_pos, int K);

// ---- indexer scan ------------------------------------------------------------------------
// Scores of query rows r = (seq, query) against their candidates, written to
// scores[r * score_stride + j] for candidate position j; fp32. Also writes
// n_vis[r] (visible entries) and count[r] (candidate positions considered).
struct ScanArgs {
  int dt;
  const void* q;          // [rows, H, d]
  const float* w;         // [rows, H]
  const void* keys;       // [n_seq, e_cap, d]; MXFP4 codes [n_seq, e_cap, d / 2] when
  const uint8_t* key_scales;  // ... key_scales [n_seq, e_cap, d / 32] is non-null
  const int64_t* q_pos;   // [rows]
  const int32_t* e_count; // [n_seq] or null
  const int32_t* cand;    // [rows, n_cand] or null
  int64_t n_cand;
  int64_t n_seq, n_q, e_cap;
  int H, d, m;
  float* scores;          // [rows, score_stride]
  int64_t score_stride;
  int32_t* n_vis;         // [rows]
  int32_t* count;         // [rows]
  uint32_t* gmax;         // [rows, gmax_stride]: order key of the max of positions [16j, 16j+16)
  int64_t gmax_stride;
  // Decode step (rows are sequences) with its ingest split between the scan and the select
  // (ingest.pos non-null): the scan pools the indexer key of the entry the token completes;
  // the select's ingest workgroups do the rest. Only when scan_fuses_ingest() holds.
  IngestArgs ingest;
  SegArgs seg;            // decode scan without candidates: candidate segments (optional)
  int score_bf16;         // the stream scan rounds every score to bf16 before it leaves
  // with MXFP4 keys: the query is quantised to MXFP4 too (the keys' rule, per head and 32
  // channels) and the products are taken between the FP4 values
  int q_fp4;
};
// ev_start / ev_stop (both or neither): the start and stop events of the scan kernel's own
// dispatch (a scan is one kernel).
hipError_t launch_scan(const ScanArgs& a, hipStream_t s, hipEvent_t ev_start = nullptr,
                       hipEvent_t ev_stop = nullptr);
// The many-query scan (prefill) for bf16 64 x 128: pq (8 or 12) query rows and
// keys_per_block keys per workgroup, grid (key blocks, query groups).
hipError_t launch_scan_prefill(const ScanArgs& a, int pq, int keys_per_block, dim3 grid,
                               hipStream_t s, hipEvent_t e0, hipEvent_t e1);
// Whether the decode scan for this shape takes the indexer-key part of the ingest.
bool scan_fuses_ingest(int dt, int H, int d, int m);
// Whether the stream scan serves this shape, the one that reads MXFP4 keys and rounds scores
// to bf16 (bf16 queries, 64 heads x 128, one or a few query rows per sequence, no candidate
// list).
bool scan_reads_mxfp4(int dt, int H, int d, int64_t n_q, bool cand);

// ---- per-head RMSNorm and partial RoPE (norm_rope.hip) ------------------------------------
// x, out [n_rows, n_heads, dim]; flags 1 RMSNorm (gamma [dim]), 2 RoPE on the last rope_dim
// channels at pos[row], 4 with -pos
hipError_t launch_norm_rope(int dt, const void* x, const void* gamma, const int64_t* pos,
                            void* out, int64_t n_rows, int n_heads, int dim, int rope_dim,
                            float base, float eps, int flags, hipStream_t s);

// ---- FP8 main-cache entries (kv_fp8.hip) ---------------------------------------------------
// x [n_rows, 512] (T) -> entries [n_rows, 576] bytes; entries -> bf16 [n_rows, 512]
hipError_t launch_quantize_kv_fp8(int dt, const void* x, void* out, int64_t n_rows,
                                  hipStream_t s);
hipError_t launch_dequantize_kv_fp8(const void* in, void* out, int64_t n_rows, hipStream_t s);

// ---- FP4 main-cache entries (kv_fp4.hip) ---------------------------------------------------
// x [n_rows, 512] (T) -> entries [n_rows, 288] bytes; entries -> bf16 [n_rows, 512]
hipError_t launch_quantize_kv_fp4(int dt, const void* x, void* out, int64_t n_rows,
                                  hipStream_t s);
hipError_t launch_dequantize_kv_fp4(const void* in, void* out, int64_t n_rows, hipStream_t s);

// ---- MXFP4 storage of indexer keys (mxfp4.hpp) --------------------------------------------
// x [n_rows, dim] (dim % 32 == 0) -> codes [n_rows, dim / 2] bytes, scales [n_rows, dim / 32]
hipError_t launch_quantize_mxfp4(int dt, const void* x, void* codes, void* scales, int64_t n_rows,
                                 int dim, hipStream_t s);

// ---- selection ---------------------------------------------------------------------------
// Top-K of each row's `count[r]` positions; position j has score scores[r*stride + j] and
// id (ids ? ids[r*id_stride + j] : j); an id is valid iff 0 <= id < id_limit[r] (or id >= 0
// when id_limit is null); ids must ascend with position. Result ids ascending, -1 padded,
// in out_idx[r*out_stride + k]. gmax (optional) holds the order keys of the maxima of 16
// consecutive scores.
struct TopkArgs {
  const float* scores;
  int64_t stride;
  const uint32_t* gmax;   // order keys of 16-position maxima (optional)
  int64_t gstride;
  const int32_t* ids;
  int64_t id_stride;
  const int32_t* id_limit;
  const int32_t* count;
  int64_t rows;
  int64_t max_count;      // upper bound of count[r] (sizes the launch)
  int K;
  int32_t* out_idx;
  float* out_score;       // may be null
  int64_t out_stride;
  void* scratch;          // segment buffers (see topk_scratch_bytes)
  // optional: the rest of a decode step's ingest (tails, rings, main entry), run by extra
  // workgroups of the select's last launch (indexer keys are the scan's part)
  const IngestArgs* side;
  SegArgs seg;            // segments left by the scan (seg.seg non-null: the select uses them)
  bool bf16_scores;       // every score is a bf16 value (the scan rounded them)
};
size_t topk_scratch_bytes(int64_t rows, int64_t max_count, int K);

hipError_t launch_topk(const TopkArgs& a, hipStream_t s);

// Block maxima of each row's first count[r] scores; nb[r] = ceil(count/bs).
hipError_t launch_block_max(const float* scores, int64_t stride, const int32_t* count,
                            int64_t rows, int64_t max_count, int bs, float* bmax,
                            int64_t bmax_stride, int32_t* nb, hipStream_t s);
// Pool of the selected blocks (ascending block ids, -1 padded): entries b*bs.. below n_vis.
hipError_t launch_pool_build(const int32_t* blocks, int64_t rows, int max_blocks, int bs,
                             const int32_t* n_vis, int32_t* pool, hipStream_t s);

// Expand a row's scores to the caller's scores_all layout (non-candidates -inf).
hipError_t launch_fill_scores(const float* scores, int64_t stride, const int32_t* count,
                              int64_t rows, int64_t n_keys, float* out, hipStream_t s);

// ---- sparse attention --------------------------------------------------------------------
struct AttnArgs {
  int dt;
  const void* q;          // [rows, H, D]
  const void* kv;         // [n_seq, e_cap, D]
  const int32_t* idx;     // [rows, top_k]
  int top_k;
  const void* win;        // [n_seq, w_cap, D]
  int w_cap, window;
  const int64_t* q_pos;   // [rows]
  const float* sink;      // [H] or null
  float scale;
  void* out;              // [rows, H, D]
  int64_t n_seq, n_q, e_cap;
  int H, D;
  void* ws;
  // inverse RoPE on the output: the last out_rope_dim channels of each head rotate in pairs
  // (2j, 2j+1) by -q_pos * base^(-2j/out_rope_dim) before the store (0: off)
  int out_rope_dim;
  double rope_log2_base;
  // how kv holds its entries: kKvPlain (T, D channels), kKvFp8 (576 bytes: 448 E4M3 + 64 bf16
  // channels) or kKvFp4 (288 bytes: E2M1 + an E4M3 scale per 16 channels); the quantised forms
  // for bf16 64 x 512 heads only
  int kv_fmt;
};
size_t attn_ws_bytes(int64_t rows, int H, int D, int top_k, int window, int dt);
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);
// merge of the split partials that launch_attn left in a.ws
hipError_t launch_attn_combine(const AttnArgs& a, int nsplit, hipStream_t s);

}  // namespace csa
