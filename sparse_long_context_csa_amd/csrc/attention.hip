// Sparse attention over selected compressed entries + the local window, with a per-head sink.
//
// "DeepSeek V4-Flash: The Cost of Deciding What to Read": section "Key and value are the
// same vector" (one cached row serves as key and value for all heads, multi-query style);
// "Attention sink, and heads that abstain" (exp(z'_h) joins the softmax denominator and
// nothing else); "The sliding window is not an optimisation" (window rows concatenated with
// the selected entries before the softmax). "DeepSeek-V4.1-Flash's KV-Cache Compression,
// Checked Down to the Byte", section 5: a query at i reads window rows [i-W+1, i].
//
// attn_mfma_kernel (bf16, 64 heads x 512): a workgroup of 4 waves (16 heads each) walks the
// row list of one query (selected ids, then window positions) in tiles of 32 rows. Each
// tile is gathered once from HBM into LDS twice: row-major (A operand of S^T = KV.Q^T,
// v_mfma_f32_16x16x32_bf16, M = 32 rows, N = 16 heads, K = 512) and transposed (B operand
// of O = P.V, K = 32 rows). The score accumulator layout puts, in every lane, 8 rows of one
// head; those 8 rows are exactly the lane's K slots of the P.V product, so P goes from the
// score registers to the A operand with no data movement. Online softmax in base 2.
// Few query rows (decode): the row list is split over workgroups; partial (max, sum,
// unnormalised output, the output in bf16 to halve what is written and read back) go to the
// workspace and attn_combine_kernel merges them in split order (deterministic).
// attn_generic_kernel covers fp32 and other head shapes.
#include <stdlib.h>

#include "attn_core.hpp"
#include "csa_common.hpp"
#include "launch.hpp"

namespace csa {

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Row j of a query's list: j < top_k -> selected id; else window position. With FP8 or FP4
// entries (kv_fmt) the pointer of a selected row is the entry's first byte.
template <typename T>
__device__ __forceinline__ const T* row_ptr(const AttnArgs& a, int64_t r, int64_t sq, int64_t t,
                                            int64_t j, int nrows) {
  if (j >= nrows) return nullptr;
  if (j < a.top_k) {
    const int32_t id = a.idx[r * a.top_k + j];
    if (id < 0 || id >= a.e_cap) return nullptr;
    if (a.kv_fmt != kKvPlain)   // a quantised entry; the kernels that take one read bytes
      return reinterpret_cast<const T*>(static_cast<const uint8_t*>(a.kv) +
                                        (sq * a.e_cap + id) *
                                            (a.kv_fmt == kKvFp8 ? kFp8EntryBytes : kFp4EntryBytes));
    return reinterpret_cast<const T*>(a.kv) + (sq * a.e_cap + id) * a.D;
  }
  const int64_t p = t - a.window + 1 + (j - a.top_k);
  if (p < 0 || p > t) return nullptr;
  return reinterpret_cast<const T*>(a.win) + (sq * a.w_cap + p % a.w_cap) * a.D;
}

}  // namespace

// Number of row splits per query row (workgroups sharing one query's rows): few query rows
// (decode) spread each row list over up to 256 workgroups in all, one tile or more each:
// a wave's chain of LDS reads and MFMAs per tile is latency-bound, so tiles run in
// parallel workgroups and the partial results are merged afterwards.
constexpr int kMinTilesPerSplit = 1;
static int attn_tune(const char* name, int dflt) {
  const char* v = getenv(name);
  return v ? atoi(v) : dflt;
}
static int attn_splits(int64_t rows, int top_k, int window, int H, int D, int dt) {
  if (!(dt == kBF16 && H == kAH && D == kAD)) return 1;
  const int64_t tiles = ceil_div(int64_t(top_k) + window, kTile);
  if (rows >= 256 || tiles < 2) return 1;
  static const int min_tiles = attn_tune("CSA_TUNE_ATTN_MIN_TILES", kMinTilesPerSplit);
  static const int total = attn_tune("CSA_TUNE_ATTN_WGS", 256);
  int64_t want = ceil_div(tiles, min_tiles > 0 ? min_tiles : kMinTilesPerSplit);
  const int64_t cap = (total > 0 ? total : 256) / rows;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  // the longest split sets the time: as few splits as give that length (8,320 rows over 64
  // splits take 5 tiles each, and 52 splits do it), so none is empty and fewer partials merge
  return int(ceil_div(tiles, ceil_div(tiles, want)));
}

size_t attn_ws_bytes(int64_t rows, int H, int D, int top_k, int window, int dt) {
  const int ns = attn_splits(rows, top_k, window, H, D, dt);
  if (ns <= 1) return 0;
  return size_t(rows) * ns * (kPartO * 2 + kAH * 8);   // bf16 outputs, fp32 (max, sum)
}

__global__ __launch_bounds__(256) void attn_mfma_kernel(AttnArgs a, int nsplit, int tiles_per_split) {
  __shared__ AttnLds lds;
  const int64_t r = blockIdx.y;
  const int64_t sq = r / a.n_q;
  const int64_t t = a.q_pos[r];
  attn_split_mfma(a, lds, r, blockIdx.x, nsplit, tiles_per_split, gridDim.y,
                  [&](int64_t j, int nrows) { return row_ptr<uint16_t>(a, r, sq, t, j, nrows); });
}

__global__ __launch_bounds__(256, 2) void attn_dma_kernel(AttnArgs a, int nsplit, int tiles_per_split) {
  __shared__ AttnDmaLds lds;
  const int64_t r = blockIdx.y;
  const int64_t sq = r / a.n_q;
  const int64_t t = a.q_pos[r];
  attn_split_dma(a, lds, r, blockIdx.x, nsplit, tiles_per_split, gridDim.y,
                 [&](int64_t j, int nrows) { return row_ptr<uint16_t>(a, r, sq, t, j, nrows); });
}

// Merge the row splits. Grid (32, rows): workgroup x covers the heads of accumulator wave
// w = x / 8 and the dims of 4 accumulator columns; its threads compute the split weights
// e^{m_s - M} of those 16 heads into LDS (16 threads per head, each over every 16th split),
// then every thread sums its 4 heads x 1 dim over the splits in split order with independent
// loads and scales by 1 / den.
constexpr int kMaxSplit = 256;

// kSplitRegs: partials held per thread in the first load round (32, or 64 when a row has more
// than 32 splits, so that up to 64 merge after one round trip).
template <int kSplitRegs>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, int nsplit) {
  __shared__ float wgt[kMaxSplit][16];
  __shared__ float2 mls[kMaxSplit][16];
  __shared__ float red[16][16];
  __shared__ float inv[16];
  const int64_t r = blockIdx.y;
  const int w = blockIdx.x >> 3;
  const int nt = (blockIdx.x & 7) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t rows = gridDim.y;
  const float2* ml = part_ml(a.ws, rows * nsplit, r * nsplit);
  const uint2* part = part_out(a.ws, r * nsplit) + (w * 32 + nt) * kWave + lane;
  constexpr int64_t sstride = kPartO / 4;   // 8-byte cells per split
  // the (max, sum) pairs of the first kSplitRegs splits and their partials load first,
  // all in one round: no load is masked (indices past the last split read the last one, whose
  // value is then ignored), so none waits for another
  constexpr int kMlRegs = kSplitRegs / 16;
  const int nml = nsplit * 16;
  float2 mlv[kMlRegs];
#pragma unroll
  for (int i = 0; i < kMlRegs; ++i) {
    const int q0 = int(threadIdx.x) + i * 256, q = q0 < nml ? q0 : nml - 1;
    mlv[i] = ml[(q >> 4) * kAH + 16 * w + (q & 15)];
  }
  uint2 v[kSplitRegs];
#pragma unroll
  for (int sp = 0; sp < kSplitRegs; ++sp) v[sp] = part[(sp < nsplit ? sp : nsplit - 1) * sstride];
  // the sink logit of this thread's head in the weights below, loaded behind them
  const float sink_l = a.sink ? a.sink[16 * w + (threadIdx.x & 15)] : 0.f;
#pragma unroll
  for (int i = 0; i < kMlRegs; ++i) {
    const int q = int(threadIdx.x) + i * 256;
    if (q < nml) mls[q >> 4][q & 15] = mlv[i];
  }
  for (int q = int(threadIdx.x) + kMlRegs * 256; q < nml; q += 256)
    mls[q >> 4][q & 15] = ml[(q >> 4) * kAH + 16 * w + (q & 15)];
  __syncthreads();
  // split weights e^(m_s - M) of the 16 heads: thread (group k, head hl) takes splits k, k + 16,
  // ...; the maxima and the denominators' partial sums meet in red (fixed order: the result
  // does not depend on scheduling). The 1 / denominator multiplies the sums at the end.
  {
    const int hl = threadIdx.x & 15, k = threadIdx.x >> 4;
    float mloc = neg_inf();
    for (int sp = k; sp < nsplit; sp += 16) mloc = fmaxf(mloc, mls[sp][hl].x);
    red[k][hl] = mloc;
    __syncthreads();
    const float zs = a.sink ? sink_l * kLog2e : neg_inf();
    float M = zs;
#pragma unroll
    for (int j = 0; j < 16; ++j) M = fmaxf(M, red[j][hl]);
    __syncthreads();   // every thread has its maximum before red holds the sums
    float dloc = 0.f;
    for (int sp = k; sp < nsplit; sp += 16) {
      const float2 m2 = mls[sp][hl];
      const float e = (m2.x == neg_inf() || M == neg_inf()) ? 0.f : exp2f(m2.x - M);
      wgt[sp][hl] = e;
      dloc += m2.y * e;
    }
    red[k][hl] = dloc;
    __syncthreads();
    if (threadIdx.x < 16) {
      float den = (zs == neg_inf() || M == neg_inf()) ? 0.f : exp2f(zs - M);
#pragma unroll
      for (int j = 0; j < 16; ++j) den += red[j][hl];
      inv[hl] = den > 0.f ? 1.f / den : 0.f;
    }
    __syncthreads();
  }
  const int g = lane >> 4, col = lane & 15;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  auto add = [&](const uint2 c, int sp) {
    const float x[4] = {bf16_to_f32(uint16_t(c.x & 0xffffu)), bf16_to_f32(uint16_t(c.x >> 16)),
                        bf16_to_f32(uint16_t(c.y & 0xffffu)), bf16_to_f32(uint16_t(c.y >> 16))};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(x[i], wgt[sp][4 * g + i], acc[i]);
  };
#pragma unroll
  for (int sp = 0; sp < kSplitRegs; ++sp)
    if (sp < nsplit) add(v[sp], sp);
  // further splits in chunks of kSplitRegs, each chunk's loads issued together
  for (int s0 = kSplitRegs; s0 < nsplit; s0 += kSplitRegs) {
#pragma unroll
    for (int k = 0; k < kSplitRegs; ++k) v[k] = part[(s0 + k < nsplit ? s0 + k : nsplit - 1) * sstride];
#pragma unroll
    for (int k = 0; k < kSplitRegs; ++k)
      if (s0 + k < nsplit) add(v[k], s0 + k);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] *= inv[4 * g + i];
  uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + (r * kAH + 16 * w + 4 * g) * kAD + nt * 16 + col;
  if (a.out_rope_dim > 0 && nt * 16 >= kAD - a.out_rope_dim) {   // uniform over the wave
    const int d = nt * 16 + col;
    float c, sn;
    rope_cos_sin(-double(a.q_pos[r]), (d - (kAD - a.out_rope_dim)) >> 1, a.out_rope_dim,
                 a.rope_log2_base, c, sn);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = rope_pair_lane(acc[i], (col & 1) != 0, c, sn);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) op[i * kAD] = f32_to_bf16(acc[i]);
}

// ---- generic: one wave per (row, head); lanes hold 8 dims each --------------------------
template <typename T>
__global__ __launch_bounds__(256) void attn_generic_kernel(AttnArgs a) {
  const int64_t r = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (h >= a.H) return;
  const int D = a.D;
  const int64_t sq = r / a.n_q;
  const int64_t t = a.q_pos[r];
  const int nrows = a.top_k + a.window;
  const int c0 = lane * 8;
  const bool act = c0 < D;
  float q[8] = {0, 0, 0, 0, 0, 0, 0, 0}, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (act) Elt<T>::load8(reinterpret_cast<const T*>(a.q) + (r * a.H + h) * D + c0, q);
  const float sl2 = a.scale * kLog2e;
  float m_run = neg_inf(), l_run = 0.f;
  for (int j = 0; j < nrows; ++j) {
    const T* src = row_ptr<T>(a, r, sq, t, j, nrows);
    if (src == nullptr) continue;
    float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (act) Elt<T>::load8(src + c0, v);
    float d = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) d = fmaf(q[c], v[c], d);
    const float s = wave_sum(d) * sl2;
    const float m_new = fmaxf(m_run, s);
    const float alpha = exp2f(m_run - m_new);
    const float pj = exp2f(s - m_new);
    l_run = l_run * alpha + pj;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = acc[c] * alpha + pj * v[c];
    m_run = m_new;
  }
  const float zs = a.sink ? a.sink[h] * kLog2e : neg_inf();
  const float M = fmaxf(m_run, zs);
  float f = 0.f;
  if (M != neg_inf()) {
    const float em = (m_run == neg_inf()) ? 0.f : exp2f(m_run - M);
    const float den = l_run * em + ((zs == neg_inf()) ? 0.f : exp2f(zs - M));
    f = den > 0.f ? em / den : 0.f;
  }
  if (act) {
    float o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = acc[c] * f;
    if (a.out_rope_dim > 0) {
      const int r0 = D - a.out_rope_dim;
#pragma unroll
      for (int c = 0; c < 8; c += 2)
        if (c0 + c >= r0) {
          float cs, sn;
          rope_cos_sin(-double(t), (c0 + c - r0) >> 1, a.out_rope_dim, a.rope_log2_base, cs, sn);
          const float x0 = o[c], x1 = o[c + 1];
          o[c] = x0 * cs - x1 * sn;
          o[c + 1] = x0 * sn + x1 * cs;
        }
    }
    Elt<T>::store8(reinterpret_cast<T*>(a.out) + (r * a.H + h) * D + c0, o);
  }
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  const int64_t rows = a.n_seq * a.n_q;
  if (rows == 0) return hipSuccess;
  const bool fast = a.dt == kBF16 && a.H == kAH && a.D == kAD;
  if (!fast) {
    const dim3 grid(unsigned((a.H + 3) / 4), unsigned(rows));
    if (a.dt == kBF16) hipLaunchKernelGGL(attn_generic_kernel<uint16_t>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(attn_generic_kernel<float>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const int ns = attn_splits(rows, a.top_k, a.window, a.H, a.D, a.dt);
  const int64_t tiles = ceil_div(int64_t(a.top_k) + a.window, kTile);
  const int tps = int(ceil_div(tiles > 0 ? tiles : 1, ns));
  const dim3 grid(static_cast<unsigned>(ns), static_cast<unsigned>(rows));
  if (int64_t(tps) * kTile <= kMaxRowsLds)
    hipLaunchKernelGGL(attn_dma_kernel, grid, dim3(256), 0, s, a, ns, tps);
  else
    hipLaunchKernelGGL(attn_mfma_kernel, grid, dim3(256), 0, s, a, ns, tps);
  if (ns > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_attn_combine(a, ns, s);
  }
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, int nsplit, hipStream_t s) {
  const int64_t rows = a.n_seq * a.n_q;
  const dim3 g2(32u, static_cast<unsigned>(rows));
  if (nsplit > 32) hipLaunchKernelGGL(attn_combine_kernel<64>, g2, dim3(256), 0, s, a, nsplit);
  else hipLaunchKernelGGL(attn_combine_kernel<32>, g2, dim3(256), 0, s, a, nsplit);
  return hipGetLastError();
}

}  // namespace csa
