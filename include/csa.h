/*
 * libcsa -- the Compressed Sparse Attention (CSA) hot path for AMD MI355X (gfx950).
 *
 * Sources (page titles and the sections each call follows):
 *   [CoD]  "DeepSeek V4-Flash: The Cost of Deciding What to Read" (The Software Frontier)
 *   [B890] "DeepSeek-V4.1-Flash's KV-Cache Compression, Checked Down to the Byte" (flozi-tech)
 *   [V41]  "DeepSeek-V4.1-Flash" interactive architecture study (shuhuayu.github.io)
 *
 * Conventions shared by every call:
 *   - Tensor pointers are DEVICE pointers to dense row-major arrays (no strides unless an
 *     argument says so). Scalars and the descriptor struct of csa_decode_step live on the
 *     host; the pointers inside it are device pointers.
 *   - dtype selects the storage type of the floating tensors documented as "T": CSA_BF16
 *     (bfloat16) or CSA_F32. Gates (w), sinks and scores are always fp32; ids int32;
 *     positions int64. Arithmetic is fp32 throughout; stored results are rounded to T by
 *     round-to-nearest-even.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream). Arguments are validated on the host before anything is launched:
 *     a call that returns an error launched nothing. CSA_ERR_HIP reports a failed launch.
 *     Outputs are valid once the stream has reached the call.
 *   - The library never allocates or frees device memory. Scratch space is the caller's
 *     workspace `ws` of at least the bytes the matching *_workspace_size call returns
 *     (256-byte aligned). A workspace must not be shared by calls that may run concurrently.
 *     Calls are thread-safe. The one exception is csa_decode_step_noalloc: its workspace is a
 *     static device array per GPU, kept until the process ends and shared by every call of it
 *     on that GPU.
 *   - Values that live on the device (positions, entry counts, ids) cannot be checked on
 *     the host; kernels clamp them so that no access leaves the documented buffers:
 *     visible counts are capped at the cache capacity, out-of-range ids are skipped.
 */
#ifndef LIBCSA_CSA_H
#define LIBCSA_CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 16

typedef enum { CSA_F32 = 0, CSA_BF16 = 1 } csa_dtype;

typedef enum {
  CSA_OK = 0,
  CSA_ERR_NULL = -1,        /* a required pointer is NULL                              */
  CSA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent                  */
  CSA_ERR_DTYPE = -3,       /* unknown dtype                                           */
  CSA_ERR_UNSUPPORTED = -4, /* valid request outside this build's limits               */
  CSA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required              */
  CSA_ERR_HIP = -6          /* a HIP launch failed                                     */
} csa_status;

/* Version of this header's ABI (CSA_ABI_VERSION). */
int csa_abi_version(void);

/* Static, NUL-terminated description of a status code (host memory, never freed). */
const char *csa_status_str(int status);

/* ---------------------------------------------------------------------------------------
 * csa_compress -- learned channel-wise softmax pooling (one stream).
 *   [CoD "The compressor has two streams and they overlap": per-channel softmax over the
 *   pooled positions, weighted sum of the rows; CoD CSA/HCA layer tables: positional bias
 *   of shape m x d; V41 "CSA2: separate producing, selecting, and reading": groups pooled
 *   by a channel-wise softmax, no overlap.]
 * For every sequence s, entry e < n_tok/m and channel c:
 *   a_j = logits[s, e*m+j, c] + bias[j, c]   (j < m),   alpha = softmax_j(a)
 *   out[s, e, c] = sum_j alpha_j * x[s, e*m+j, c]
 *   x, logits : T [n_seq, n_tok, dim]      bias : T [m, dim]
 *   out       : T, entry e of sequence s at out + s*out_seq_stride + e*dim
 *               (out_seq_stride = 0 means dense: (n_tok/m)*dim). Writing into a cache at
 *               an entry offset is done by offsetting `out` and passing the cache stride.
 * Limits: 1 <= m <= 128 (HCA pools m' = 128: [CoD] "Heavily Compressed Attention"),
 * n_tok % m == 0, 8 <= dim <= 8192, dim % 8 == 0.
 * ------------------------------------------------------------------------------------- */
int csa_compress(const void *x, const void *logits, const void *bias, void *out,
                 int64_t n_seq, int64_t n_tok, int64_t out_seq_stride, int32_t dim,
                 int32_t m, int32_t dtype, void *stream);

/* ---------------------------------------------------------------------------------------
 * csa_compress_c4a -- the overlapped two-stream compressor (vLLM's "c4a" at m = 4).
 *   [CoD "The compressor has two streams and they overlap": two independent projections C^a
 *   and C^b with their own compression logits; entry i draws C^a from the positions of its
 *   own block and C^b from the block before, one softmax across the 2m logits per channel,
 *   a weighted sum over both streams (eight tokens at stride four for m = 4); CoD CSA layer
 *   table: positional biases B^a, B^b of shape m x d.]
 * For every sequence s, chunk entry e < n_tok/m and channel c, with j < m:
 *   logits = { za[s, m e + j, c] + bias_a[j, c] }  U  { zb'[s, j, c] + bias_b[j, c] }
 *   alpha  = softmax over all 2m of them
 *   out[s, e, c] = sum of alpha times xa[s, m e + j, c] and xb'[s, j, c] respectively
 * where (xb', zb') are the b-stream rows of the block before: rows m(e-1) + j of xb, zb for
 * e > 0, and for e = 0 rows j of xb_prev, zb_prev -- or, when both are NULL (the chunk starts
 * the sequence), no b-part: entry 0 of a sequence pools its m a-rows only.
 *   xa, za, xb, zb : T [n_seq, n_tok, dim]  rows of positions p0 .. p0 + n_tok - 1
 *                    (p0 a multiple of m: the chunk starts on a block boundary)
 *   bias_a, bias_b : T [m, dim]
 *   xb_prev, zb_prev : T [n_seq, m, dim] the b rows of positions p0 - m .. p0 - 1, or NULL
 *   out            : T, chunk entry e of sequence s at out + s*out_seq_stride + e*dim
 *                    (out_seq_stride = 0 means dense: (n_tok/m)*dim)
 * Limits: as csa_compress (1 <= m <= 16, n_tok % m == 0, 8 <= dim <= 8192, dim % 8 == 0);
 * xb_prev and zb_prev both NULL or both set (else CSA_ERR_NULL).
 * ------------------------------------------------------------------------------------- */
int csa_compress_c4a(const void *xa, const void *za, const void *xb, const void *zb,
                     const void *bias_a, const void *bias_b, const void *xb_prev,
                     const void *zb_prev, void *out, int64_t n_seq, int64_t n_tok,
                     int64_t out_seq_stride, int32_t dim, int32_t m, int32_t dtype,
                     void *stream);

/* ---------------------------------------------------------------------------------------
 * csa_norm_rope -- per-head RMSNorm and partial RoPE in one pass.
 *   [CoD "Key and value are the same vector": RMSNorm per head on the queries and on the
 *   single head of the compressed KV entries just before the core attention; RoPE on the last
 *   64 dimensions of each head; RoPE with position -i on each head's output undoes the
 *   rotation a shared key/value carries.]
 * For row r, head h and vector v = x[r, h, :] (dim channels):
 *   flags & CSA_NR_NORM:    v <- v / sqrt(mean(v^2) + eps) * gamma
 *   flags & CSA_NR_ROPE:    the last rope_dim channels rotate in pairs (2j, 2j+1) (counted from
 *                           channel dim - rope_dim) by the angle p * rope_base^(-2j/rope_dim),
 *                           p = pos[r], or p = -pos[r] with CSA_NR_INVERSE as well
 *   out[r, h, :] <- v (rounded once to T; out may be x)
 *   x, out : T [n_rows, n_heads, dim]    gamma : T [dim] (with CSA_NR_NORM) or NULL
 *   pos    : i64 [n_rows] (with CSA_NR_ROPE) or NULL
 * Limits: 8 <= dim <= 512, dim % 8 == 0; 0 <= rope_dim <= dim, rope_dim even; rope_base > 1;
 * eps >= 0; flags within the three bits.
 * ------------------------------------------------------------------------------------- */
#define CSA_NR_NORM 1
#define CSA_NR_ROPE 2
#define CSA_NR_INVERSE 4
int csa_norm_rope(const void *x, const void *gamma, const int64_t *pos, void *out,
                  int64_t n_rows, int32_t n_heads, int32_t dim, int32_t rope_dim,
                  float rope_base, float eps, int32_t flags, int32_t dtype, void *stream);

/* ---------------------------------------------------------------------------------------
 * csa_quantize_mxfp4 -- MXFP4 storage of indexer keys (production precision).
 *   [CoD "What the cache costs, checked four ways": the indexer cache is FP4, 64 bytes per
 *   128-channel key; CoD "FP4, down to the index scores": 1 x 32 MXFP4 sub-blocks.]
 * Elements E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1,
 * 1.5, 2, 3, 4, 6), one E8M0 scale 2^(s - 127) per 32 consecutive channels. For each block:
 * s = floor(log2 max|x|) - 2 clamped to [-127, 127] (-127 for an all-zero block); each x / 2^s
 * rounds to the nearest magnitude, ties to the even code, magnitudes past 6 to 6; a zero
 * magnitude is code 0.
 *   x      : T [n_rows, dim]             (dtype CSA_BF16 or CSA_F32)
 *   codes  : uint8 [n_rows, dim / 2]     element 2i in the low nibble of byte i
 *   scales : uint8 [n_rows, dim / 32]    the bytes s
 * Limits: 32 <= dim <= 8192, dim % 32 == 0. Device pointers; asynchronous on `stream`.
 * ------------------------------------------------------------------------------------- */
int csa_quantize_mxfp4(const void *x, void *codes, void *scales, int64_t n_rows, int32_t dim,
                       int32_t dtype, void *stream);

/* ---------------------------------------------------------------------------------------
 * csa_quantize_kv_fp8 / csa_dequantize_kv_fp8 -- FP8 storage of main KV entries.
 *   [CoD "What the cache costs, checked four ways": the 64 rotary dimensions of a shared
 *   key/value entry stay in bf16 and the other 448 go to FP8: 64 * 2 + 448 = 576 bytes per
 *   512-dim entry; CoD "The indexer is O(n), and that is the ceiling": the main
 *   attention runs in FP8.]
 * Entry layout (CSA_KV_FP8_BYTES = 576): bytes 0..447 are the E4M3 codes of channels 0..447,
 * bytes 448..575 channels 448..511 as little-endian bf16 (nearest-even). E4M3 is the OCP
 * format (sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities; S.1111.111 is
 * NaN, so the largest finite magnitude is 448; exponent field 0: subnormals m * 2^-9). Each
 * value rounds to the nearest E4M3 value, ties to the even code, magnitudes past 448 to 448; a
 * zero magnitude is code 0x00. There is no scale.
 *   quantize:   x T [n_rows, 512] (CSA_BF16 or CSA_F32, rounded directly) -> out uint8
 *               [n_rows, 576] (16-byte aligned)
 *   dequantize: in uint8 [n_rows, 576] -> out bf16 [n_rows, 512] (exact: every E4M3 value is a
 *               bf16 value)
 * Device pointers; asynchronous on `stream`.
 * ------------------------------------------------------------------------------------- */
#define CSA_KV_FP8_BYTES 576

/* ---------------------------------------------------------------------------------------
 * csa_quantize_kv_fp4 / csa_dequantize_kv_fp4 -- FP4 storage of main KV entries.
 *   [B890 section 4, Cell 3 "FP4 range analysis": E2M1 elements with one E4M3 scale per 16
 *   channels and no second-level global scale, 512 x 0.5 + 512 / 16 = 288 bytes per 512-channel
 *   entry; V41 "FP4 main KV": the whole latent is quantised after RoPE, and attention
 *   dequantises the cached values before it uses them.]
 * Entry layout (CSA_KV_FP4_BYTES = 288): bytes 0..255 hold the E2M1 codes (sign, 2 exponent
 * bits with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), channel 2i in the
 * low nibble of byte i; byte 256 + g holds the E4M3 scale code of channels 16g .. 16g+15 (the
 * E4M3 of csa_quantize_kv_fp8). Per block: the scale is the E4M3 value nearest to max|x| / 6,
 * ties to the even code, past 448 to 448; a block whose scale is 0 stores all codes 0;
 * otherwise each x / scale rounds to the nearest magnitude, ties to the even code, past 6 to 6,
 * and a zero magnitude is code 0. A stored value (element x scale) is exactly a bf16 value.
 *   quantize:   x T [n_rows, 512] (CSA_BF16 or CSA_F32, rounded directly) -> out uint8
 *               [n_rows, 288] (16-byte aligned)
 *   dequantize: in uint8 [n_rows, 288] (16-byte aligned) -> out bf16 [n_rows, 512] (16-byte
 *               aligned; exact)
 * Device pointers; asynchronous on `stream`.
 * ------------------------------------------------------------------------------------- */
#define CSA_KV_FP4_BYTES 288
int csa_quantize_kv_fp4(const void *x, void *out, int64_t n_rows, int32_t dtype, void *stream);
int csa_dequantize_kv_fp4(const void *in, void *out, int64_t n_rows, void *stream);
int csa_quantize_kv_fp8(const void *x, void *out, int64_t n_rows, int32_t dtype, void *stream);
int csa_dequantize_kv_fp8(const void *in, void *out, int64_t n_rows, void *stream);

/* ---------------------------------------------------------------------------------------
 * csa_index_topk -- lightning-indexer scores + Top-K selection.
 *   [CoD "The Lightning Indexer": I(t,s) = sum_h w(t,h) * ReLU(q_I(t,h) . K_s); keep the
 *   top k (512 in V4-Flash). CoD "The sliding window is not an optimisation": entry i is
 *   usable by a query at t only if m*(i+1)-1 <= t.]
 * For query row (s, i) at position t = q_pos[s, i]:
 *   n_vis = min(e_count[s], floor((t+1)/m), e_cap)   (0 when t < 0; e_count NULL: e_cap)
 *   candidates = entries 0..n_vis-1, or, when cand != NULL, the ids cand[s, i, 0..n_cand)
 *                that satisfy 0 <= id < n_vis (others are ignored). cand lists must be
 *                ascending (a pool from csa_index_blocks is).
 *   out_idx[s, i, :] = the min(top_k, #candidates) candidates with the highest fp32 score,
 *                ties to the lower id, written in ascending id order, padded with -1.
 *   q_idx   : T [n_seq, n_q, idx_heads, idx_dim]     w : f32 [n_seq, n_q, idx_heads]
 *   k_idx   : T [n_seq, e_cap, idx_dim]               q_pos : i64 [n_seq, n_q]
 *   e_count : i32 [n_seq] or NULL                     cand  : i32 [n_seq, n_q, n_cand] or NULL
 *   out_idx : i32 [n_seq, n_q, top_k]
 *   out_score  : f32 [n_seq, n_q, top_k] or NULL: score of each selected id (-inf for pads)
 *   scores_all : f32 [n_seq, n_q, n_keys] or NULL: every score (n_keys = n_cand if cand
 *                else e_cap); positions that are not candidates hold -inf.
 * Limits: 1 <= idx_heads <= 64, 8 <= idx_dim <= 256, idx_dim % 8 == 0,
 *   idx_heads*idx_dim <= 8192 (bf16 fast path: 64 x 128), 1 <= top_k <= 2048,
 *   1 <= m <= 16, 1 <= e_cap < 2^31, 0 <= n_cand <= 65536, n_seq*n_q <= 65535.
 * ------------------------------------------------------------------------------------- */
size_t csa_index_topk_workspace_size(int64_t n_seq, int64_t n_q, int64_t n_keys,
                                     int32_t top_k);
int csa_index_topk(const void *q_idx, const float *w, const void *k_idx,
                   const int64_t *q_pos, const int32_t *e_count, const int32_t *cand,
                   int32_t n_cand, int64_t n_seq, int64_t n_q, int64_t e_cap,
                   int32_t idx_heads, int32_t idx_dim, int32_t m, int32_t top_k,
                   int32_t *out_idx, float *out_score, float *scores_all, void *ws,
                   size_t ws_bytes, int32_t dtype, void *stream);

/* ---------------------------------------------------------------------------------------
 * csa_index_scores -- the lightning indexer's scores alone (csa_index_topk's scan, no
 * selection).
 *   [CoD "The Lightning Indexer": I(t,s) = sum_h w(t,h) * ReLU(q_I(t,h) . K_s); CoD "The
 *   sliding window is not an optimisation": entry i is usable at t only if m*(i+1)-1 <= t;
 *   CoD "The indexer is O(n), and that is the ceiling": the scan touches every visible entry.]
 * For query row r = (s, i) at t = q_pos[s, i], n_vis as in csa_index_topk (no candidate list):
 *   scores[r * score_stride + e] = I(t, e) in fp32 for 0 <= e < n_vis; the rest of the row
 *   (e >= n_vis) is not written.
 *   q_idx, w, k_idx, q_pos, e_count : as csa_index_topk
 *   scores : f32, 16-byte aligned; score_stride >= e_cap and a multiple of 4 (else
 *            CSA_ERR_SHAPE)
 *   ws     : csa_index_scores_workspace_size(n_seq, n_q, e_cap) bytes (the scan's visible
 *            counts and per-16-position maxima), not read before it is written
 * The scan is the same kernel, grid and arithmetic as inside csa_index_topk for the same
 * shapes, so the scores equal the ones that call ranks. Limits: as csa_index_topk.
 * ------------------------------------------------------------------------------------- */
size_t csa_index_scores_workspace_size(int64_t n_seq, int64_t n_q, int64_t e_cap);
int csa_index_scores(const void *q_idx, const float *w, const void *k_idx,
                     const int64_t *q_pos, const int32_t *e_count, int64_t n_seq, int64_t n_q,
                     int64_t e_cap, int32_t idx_heads, int32_t idx_dim, int32_t m,
                     float *scores, int64_t score_stride, void *ws, size_t ws_bytes,
                     int32_t dtype, void *stream);

/* ---------------------------------------------------------------------------------------
 * csa_index_blocks -- hierarchical pre-select: full scan -> block maxima -> pool.
 *   [B890 section 3: the first Full layer scores the whole visible range and selects at
 *   most 2,048 blocks of 8 positions, a pool of up to 16,384 candidates that later
 *   Reindex layers rescore. V41 "Hierarchical indexing bounds the deeper searches": each
 *   8-position block is scored by its maximum; the Full layer also takes its own Top-512.]
 * For query row (s, i) (visibility as in csa_index_topk):
 *   Bmax[b]  = max of the fp32 scores of visible entries in [b*block_size, (b+1)*block_size)
 *   blocks   = the min(max_blocks, #blocks) blocks with the highest Bmax (ties: lower b)
 *   out_pool[s, i, :] = the visible entries of those blocks, ascending, padded with -1
 *   out_idx  (optional, NULL to skip) = this row's own Top-top_k as in csa_index_topk.
 *   out_pool : i32 [n_seq, n_q, max_blocks*block_size]   out_idx : i32 [n_seq, n_q, top_k]
 * Pass out_pool as `cand` (n_cand = max_blocks*block_size) to csa_index_topk to rescore.
 * Limits: as csa_index_topk; 1 <= block_size <= 64, max_blocks >= 1,
 *   block_size*max_blocks <= 32768; 0 <= top_k <= 2048 (ignored when out_idx is NULL).
 * ------------------------------------------------------------------------------------- */
size_t csa_index_blocks_workspace_size(int64_t n_seq, int64_t n_q, int64_t e_cap,
                                       int32_t block_size, int32_t max_blocks,
                                       int32_t top_k);
int csa_index_blocks(const void *q_idx, const float *w, const void *k_idx,
                     const int64_t *q_pos, const int32_t *e_count, int64_t n_seq,
                     int64_t n_q, int64_t e_cap, int32_t idx_heads, int32_t idx_dim,
                     int32_t m, int32_t block_size, int32_t max_blocks, int32_t *out_pool,
                     int32_t top_k, int32_t *out_idx, void *ws, size_t ws_bytes,
                     int32_t dtype, void *stream);

/* ---------------------------------------------------------------------------------------
 * csa_sparse_attn -- attention over supplied selected entries + local window + sink.
 *   [CoD "Key and value are the same vector": one cached entry serves as key and value;
 *   "Attention sink, and heads that abstain": exp(z'_h) joins the softmax denominator
 *   only; "The sliding window is not an optimisation": the window rows are concatenated
 *   with the selected entries before the softmax. B890 section 5: a query at i reads the
 *   window [i-W+1, i]. V41 "What this means for existing V4 code": the attention kernel
 *   gathers local and selected global latents, takes supplied selections, normalises
 *   with the sink. CoD "Heavily Compressed Attention": top-k = all serves dense HCA.]
 * For query row (s, i) at t = q_pos[s, i] and head h:
 *   J   = { kv[s, idx[s,i,k]] : 0 <= idx[s,i,k] < e_cap }           (k < top_k; -1 skipped)
 *       + { win[s, p % w_cap] : max(0, t-window+1) <= p <= t }         (raw window rows)
 *   z_j = scale * q[s,i,h,:] . row_j
 *   out[s,i,h,:] = sum_j e^{z_j} row_j / (sum_j e^{z_j} + e^{sink[h]})   (0 when J empty)
 *   q   : T [n_seq, n_q, n_heads, head_dim]   kv : T [n_seq, e_cap, head_dim]
 *   idx : i32 [n_seq, n_q, top_k] (any order; may be NULL when top_k == 0)
 *   win : T [n_seq, w_cap, head_dim] (may be NULL when window == 0)
 *   q_pos : i64 [n_seq, n_q]   sink : f32 [n_heads] or NULL (no sink)
 *   out : T [n_seq, n_q, n_heads, head_dim]
 * Selected ids are used as given: causality of the selection is the caller's (the ids of
 * csa_index_topk are causal). The window rows for [t-window+1, t] must be in `win`.
 * Limits: 1 <= n_heads <= 64, 8 <= head_dim <= 512, head_dim % 8 == 0, 0 <= top_k <= 16384,
 *   0 <= window <= w_cap (w_cap >= 1 when window > 0), n_seq*n_q <= 65535.
 *   bf16 fast path: n_heads == 64, head_dim == 512.
 * ------------------------------------------------------------------------------------- */
size_t csa_sparse_attn_workspace_size(int64_t n_seq, int64_t n_q, int32_t n_heads,
                                      int32_t head_dim, int32_t top_k, int32_t window);
int csa_sparse_attn(const void *q, const void *kv, const int32_t *idx, int32_t top_k,
                    const void *win, int32_t w_cap, int32_t window, const int64_t *q_pos,
                    const float *sink, float scale, void *out, int64_t n_seq, int64_t n_q,
                    int64_t e_cap, int32_t n_heads, int32_t head_dim, void *ws,
                    size_t ws_bytes, int32_t dtype, void *stream);

/* csa_sparse_attn_fp8 -- csa_sparse_attn over an FP8 main cache: kv is uint8
 * [n_seq, e_cap, 576] in csa_quantize_kv_fp8's layout (16-byte aligned) and each selected
 * entry takes part at its exact value; q, the window rows, out and the arithmetic are those of
 * csa_sparse_attn. Needs dtype CSA_BF16, n_heads 64, head_dim 512 (else CSA_ERR_UNSUPPORTED);
 * the workspace is csa_sparse_attn_workspace_size's. */
int csa_sparse_attn_fp8(const void *q, const void *kv, const int32_t *idx, int32_t top_k,
                        const void *win, int32_t w_cap, int32_t window, const int64_t *q_pos,
                        const float *sink, float scale, void *out, int64_t n_seq, int64_t n_q,
                        int64_t e_cap, int32_t n_heads, int32_t head_dim, void *ws,
                        size_t ws_bytes, int32_t dtype, void *stream);

/* csa_sparse_attn_fp4 -- csa_sparse_attn over an FP4 main cache: kv is uint8
 * [n_seq, e_cap, 288] in csa_quantize_kv_fp4's layout (16-byte aligned) and each selected
 * entry takes part at its exact value (element x scale); everything else as
 * csa_sparse_attn_fp8 (same limits, same workspace).
 *   [V41 "FP4 main KV": attention dequantises the cached values before using them.] */
int csa_sparse_attn_fp4(const void *q, const void *kv, const int32_t *idx, int32_t top_k,
                        const void *win, int32_t w_cap, int32_t window, const int64_t *q_pos,
                        const float *sink, float scale, void *out, int64_t n_seq, int64_t n_q,
                        int64_t e_cap, int32_t n_heads, int32_t head_dim, void *ws,
                        size_t ws_bytes, int32_t dtype, void *stream);

/* ---------------------------------------------------------------------------------------
 * csa_decode_step -- one new token per sequence through the whole hot path.
 *   [CoD "The compressor has two streams...", "The Lightning Indexer", "Attention sink",
 *   "The sliding window is not an optimisation"; CoD "Two cache hierarchies": compressed
 *   entries in one cache, the window and the compressor's not-yet-pooled tail in a state
 *   cache; B890 section 3 / V41 "CSA2": a selection shared by several attention calls
 *   (Reuse layers), the hierarchical pool for deeper indexers.]
 * Per sequence s at position t = pos[s] (slot = t % m):
 *   1. x_new, z_new, xi_new, zi_new enter the compressor tails at row `slot`; for every
 *      attention call c with win_new[c] != NULL, win_new[c][s] enters win[c] at row
 *      t % w_cap (with kv_gamma / kv_rope_dim, RMSNorm'd and rotated at t first, like an
 *      entry: see kv_gamma below).
 *   2. If (t+1) % m == 0 the block is complete: entry e = (t+1)/m - 1 (< e_cap, else not
 *      stored) of kv <- pool(x_tail, z_tail, bias) and of k_idx <- pool(xi_tail, zi_tail,
 *      bias_i), as csa_compress with n_tok = m.
 *   3. n_vis = min(floor((t+1)/m), e_cap): the cache must hold entries 0..n_vis-1.
 *   4. Flat (block_size == 0): out_idx[s] = Top-top_k of csa_index_topk over the visible
 *      entries with (q_idx, w). Hierarchical (block_size > 0): the pool of
 *      csa_index_blocks with (q_idx, w), then the Top-top_k of the pool rescored with
 *      (q_idx2, w2).
 *   5. For c < n_attn: out[c][s] = csa_sparse_attn of q[c][s] over out_idx[s], window rows
 *      of win[c] and sink[c] (scale shared). The calls are issued one after another.
 * Pointers (device unless noted):
 *   pos i64 [n_seq]; x_new, z_new T [n_seq, dim]; xi_new, zi_new T [n_seq, idx_dim];
 *   kv T [n_seq, e_cap, dim]; k_idx T [n_seq, e_cap, idx_dim];
 *   x_tail, z_tail T [n_seq, m, dim]; xi_tail, zi_tail T [n_seq, m, idx_dim];
 *   bias T [m, dim]; bias_i T [m, idx_dim];
 *   q_idx, q_idx2 T [n_seq, idx_heads, idx_dim]; w, w2 f32 [n_seq, idx_heads]
 *   (q_idx2/w2 only when block_size > 0);
 *   q[c] T [n_seq, n_heads, dim]; win[c] T [n_seq, w_cap, dim]; win_new[c] T [n_seq, dim]
 *   or NULL; sink[c] f32 [n_heads] or NULL; out[c] T [n_seq, n_heads, dim];
 *   out_idx i32 [n_seq, top_k].
 * Limits: as the calls it is made of; 1 <= n_attn <= CSA_MAX_ATTN.
 * ------------------------------------------------------------------------------------- */
#define CSA_MAX_ATTN 4
#define CSA_DECODE_EVENTS 5
#define CSA_IDX_DTYPE 0   /* csa_decode_desc.idx_format: indexer keys in the step's dtype */
#define CSA_IDX_MXFP4 1   /* indexer keys as MXFP4 codes + scale bytes                    */
#define CSA_IDX_MXFP4_QK 2 /* MXFP4 keys, and the query quantised to MXFP4 in the scan      */
#define CSA_SCORE_F32 0   /* csa_decode_desc.score_format: rank fp32 index scores           */
#define CSA_SCORE_BF16 1  /* rank the scores rounded to bf16                               */
#define CSA_KV_DTYPE 0    /* csa_decode_desc.kv_format: main entries in the step's dtype      */
#define CSA_KV_FP8 1      /* main entries as 576-byte FP8 entries (csa_quantize_kv_fp8)       */
#define CSA_KV_FP4 2      /* main entries as 288-byte FP4 entries (csa_quantize_kv_fp4)       */
#define CSA_COMP_SINGLE 0 /* csa_decode_desc.compressor: one main stream (csa_compress)        */
#define CSA_COMP_C4A 1    /* two overlapped main streams (csa_compress_c4a)                    */

typedef struct csa_decode_desc {
  int32_t dtype;
  int32_t m, dim, n_heads, idx_heads, idx_dim;
  int32_t top_k, window, w_cap;
  int32_t block_size, max_blocks;   /* block_size 0: flat selection */
  int32_t n_attn;
  int64_t n_seq, e_cap;
  float scale;
  const int64_t *pos;
  const void *x_new, *z_new, *xi_new, *zi_new;
  void *kv, *k_idx;
  void *x_tail, *z_tail, *xi_tail, *zi_tail;
  const void *bias, *bias_i;
  const void *q_idx;
  const float *w;
  const void *q_idx2;
  const float *w2;
  const void *q[CSA_MAX_ATTN];
  void *win[CSA_MAX_ATTN];
  const void *win_new[CSA_MAX_ATTN];
  const float *sink[CSA_MAX_ATTN];
  void *out[CSA_MAX_ATTN];
  int32_t *out_idx;
  /* Optional profiling hooks: hipEvent_t handles (as void*) recorded on `stream` at the
   * phase boundaries of the step when non-NULL: [0] start, [1] after the ingest/compress
   * kernel, [2] after the (stage-1) indexer scan, [3] after the selection (incl. the
   * hierarchical stage 2), [4] after the attention calls. The caller owns the events. */
  void *events[CSA_DECODE_EVENTS];
  /* Optional: hipEvent_t handles (as void*) that the (stage-1) indexer scan kernel takes as
   * the start and stop events of its own dispatch (hipExtLaunchKernel), so that their
   * interval is that kernel's run time alone, with no marker packets around it. Both NULL or
   * both set; the caller owns them. */
  void *scan_events[2];
  /* Storage of the indexer keys: CSA_IDX_DTYPE keeps k_idx in T as above; CSA_IDX_MXFP4 keeps
   * them in csa_quantize_mxfp4's form, k_idx = codes uint8 [n_seq, e_cap, idx_dim / 2] (16-byte
   * aligned) and k_idx_scale = scale bytes uint8 [n_seq, e_cap, idx_dim / 32] (4-byte
   * aligned). The scan scores the keys' exact values; the entry a step completes is pooled,
   * rounded to T and stored quantised. MXFP4 needs T = bf16, idx_heads 64, idx_dim 128, the
   * flat selection (block_size 0) and m <= 8; otherwise CSA_ERR_UNSUPPORTED.
   * CSA_IDX_MXFP4_QK keeps the keys the same way and also takes the query into FP4: each
   * head's q_idx is quantised to MXFP4 by the keys' rule (csa_quantize_mxfp4) inside the scan,
   * and every product q . k is between the two FP4 values (exact, accumulated in fp32); the
   * ReLU, the gates and the head sum stay fp32. Same conditions as CSA_IDX_MXFP4.
   *   [CoD "What the cache costs, checked four ways": the indexer cache is FP4, 64 bytes per
   *   128-channel key; CoD "FP4, down to the index scores": the indexer's query-key path is
   *   cached, loaded and multiplied in FP4, 1 x 32 MXFP4 sub-blocks.] */
  int32_t idx_format;
  void *k_idx_scale;
  /* Precision of the index scores the selection ranks: CSA_SCORE_F32 (as in steps 4 above) or
   * CSA_SCORE_BF16, every fp32 score rounded to the nearest bf16 value (ties to even) before
   * the Top-K, ties at the K-th value still going to the lower id. CSA_SCORE_BF16 needs
   * T = bf16, idx_heads 64, idx_dim 128 and the flat selection; otherwise
   * CSA_ERR_UNSUPPORTED.
   *   [CoD "FP4, down to the index scores": the indexer's output scores are quantised from
   *   FP32 to BF16 ahead of the top-k selector.] */
  int32_t score_format;
  /* Inverse RoPE on every attention call's output: when out_rope_dim > 0, the last
   * out_rope_dim channels of each head's output rotate in pairs (2j, 2j+1) by the angle
   * -t * rope_base^(-2j/out_rope_dim) before the store (as csa_norm_rope with
   * CSA_NR_ROPE | CSA_NR_INVERSE at pos = t), fused into the attention's output store.
   * out_rope_dim even, <= dim, and a multiple of 16 for bf16 64 x 512 heads; rope_base > 1.
   *   [CoD "Key and value are the same vector": RoPE with position -i on the last 64
   *   dimensions of each head's output restores relative positions.] */
  int32_t out_rope_dim;
  float rope_base;
  /* Query preparation: q_gamma[c] (T [dim]) or NULL applies the per-head RMSNorm (eps 1e-6)
   * to call c's query; q_rope_dim > 0 then turns the last q_rope_dim channels of every head by
   * RoPE at +t (base rope_base); the prepared query (rounded to T, as csa_norm_rope stores it)
   * goes to the workspace and the call attends with it; q itself is not written. The
   * preparation runs in the workgroups of the selection launch that do the rest of the ingest
   * (off the attention's path), or as one csa_norm_rope pass per call when the ingest is a
   * kernel of its own. q_rope_dim even and at most 64, dim <= 512 (else CSA_ERR_UNSUPPORTED).
   *   [CoD "Key and value are the same vector": RMSNorm per head on the queries; RoPE on the
   *   last 64 dimensions.] */
  const void *q_gamma[CSA_MAX_ATTN];
  int32_t q_rope_dim;
  /* Storage of the main KV entries: CSA_KV_DTYPE keeps kv in T as above; CSA_KV_FP8 keeps
   * them in csa_quantize_kv_fp8's form, kv = uint8 [n_seq, e_cap, 576] (16-byte aligned): the
   * entry a step completes is pooled, rounded to T and stored as an FP8 entry, and the
   * attention reads every selected entry at its exact value. Needs T = bf16, n_heads 64 and
   * dim 512; otherwise CSA_ERR_UNSUPPORTED. CSA_KV_FP4 does the same with csa_quantize_kv_fp4's
   * form, kv = uint8 [n_seq, e_cap, 288] (16-byte aligned), under the same conditions.
   *   [CoD "What the cache costs, checked four ways": 448 FP8 + 64 bf16 rotary dims =
   *   576 bytes per entry; B890 section 4: E2M1 + one E4M3 scale per 16 channels = 288
   *   bytes per entry.] */
  int32_t kv_format;
  /* The key/value rows a step stores: kv_gamma (T [dim]) or NULL applies the per-head RMSNorm
   * (eps 1e-6) to the pooled entry; kv_rope_dim > 0 then turns its last kv_rope_dim channels by
   * RoPE at t (base rope_base), t being the position of the newest token the entry pools; the
   * result is rounded once to T (and then stored in kv_format). Every new window row
   * (win_new[c]) gets the same RMSNorm and RoPE at its position t before it enters its ring, so
   * that every row the attention reads carries its own position's rotation and the inverse
   * RoPE of the output leaves only distances. Needs dim 512; kv_rope_dim even and at most 64
   * (else CSA_ERR_UNSUPPORTED / CSA_ERR_SHAPE).
   *   [CoD "Key and value are the same vector": RMSNorm per head on the KV entries; RoPE on
   *   the last 64 dimensions, a cached row carrying its position's rotation; CoD "Two cache
   *   hierarchies, and lcm(4, 128)": vLLM fuses KV RoPE with the sliding-window key
   *   insertion.] */
  const void *kv_gamma;
  int32_t kv_rope_dim;
  /* Compressor of the main entries: CSA_COMP_SINGLE pools as step 2 above; CSA_COMP_C4A pools
   * them with the overlapped two-stream compressor. Then x_new, z_new, x_tail, z_tail and bias
   * are the a stream, and the b stream of the new token (xb_new, zb_new T [n_seq, dim]) enters
   * xb_tail, zb_tail (T [n_seq, 2m, dim]) at row t % 2m: the b rows of the last two blocks,
   * position p at row p % 2m. Entry e = (t+1)/m - 1 is then csa_compress_c4a of the a rows of
   * block e and the b rows of block e - 1 (rows ((e-1) % 2) m .. + m of xb_tail, zb_tail), with
   * bias_a = bias and bias_b (T [m, dim]); entry 0 of a sequence has no b-part. The indexer keys
   * keep the single-stream pooling of step 2. The four b pointers and bias_b are required with
   * CSA_COMP_C4A (else CSA_ERR_NULL) and ignored otherwise.
   *   [CoD "The compressor has two streams and they overlap": entry i draws C^a from its own
   *   block and C^b from the block before, one softmax over the 2m logits per channel; CoD CSA
   *   layer table: two overlapped KV streams with biases B^a, B^b.] */
  int32_t compressor;
  const void *xb_new, *zb_new;
  void *xb_tail, *zb_tail;
  const void *bias_b;
} csa_decode_desc;

size_t csa_decode_step_workspace_size(const csa_decode_desc *d);
int csa_decode_step(const csa_decode_desc *d, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------
 * csa_decode_step_noalloc -- csa_decode_step with no workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.
 * The workspace is a static device array of CSA_NOALLOC_SCRATCH_BYTES (32 MiB) inside the
 * library; every GPU the library runs on holds its own copy until the process ends. The call
 * runs the same kernels as csa_decode_step over it and never allocates or frees memory. The
 * GPU is the device of `stream` (the calling thread's current device for a NULL stream); the
 * array's device address is looked up once per device, on the first call there.
 * Errors: those of csa_decode_step; CSA_ERR_WORKSPACE when csa_decode_step_workspace_size(d)
 * exceeds CSA_NOALLOC_SCRATCH_BYTES (the 1M-context batch of 4 needs about 11 MiB, a batch of
 * 8 about 22 MiB); CSA_ERR_HIP when the array's address cannot be found.
 * Every call on one GPU shares that GPU's array, and the array keeps the last call's contents
 * (no kernel of the step needs it cleared): calls that may overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller. The descriptor's buffers are the
 * caller's as for csa_decode_step.
 * ------------------------------------------------------------------------------------- */
#define CSA_NOALLOC_SCRATCH_BYTES (32u << 20)
int csa_decode_step_noalloc(const csa_decode_desc *d, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBCSA_CSA_H */
