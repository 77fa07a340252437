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
// unnormalised output) go to the workspace and attn_combine_kernel merges them in split
// order (deterministic). attn_generic_kernel covers fp32 and other head shapes.
#include "csa_common.hpp"
#include "launch.hpp"

namespace csa {

namespace {

constexpr int kAH = 64;          // heads on the MFMA path
constexpr int kAD = 512;         // head dim on the MFMA path
constexpr int kTile = 32;        // rows per tile
constexpr int kKvRow = 1040;     // LDS bytes per row of the row-major tile (1024 + 16)
constexpr int kVtRow = 80;       // LDS bytes per dim of the transposed tile (64 + 16)

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Row j of a query's list: j < top_k -> selected id; else window position.
template <typename T>
__device__ __forceinline__ const T* row_ptr(const AttnArgs& a, int64_t r, int64_t sq, int64_t t,
                                            int64_t j, int nrows) {
  if (j >= nrows) return nullptr;
  if (j < a.top_k) {
    const int32_t id = a.idx[r * a.top_k + j];
    if (id < 0 || id >= a.e_cap) return nullptr;
    return reinterpret_cast<const T*>(a.kv) + (sq * a.e_cap + id) * a.D;
  }
  const int64_t p = t - a.window + 1 + (j - a.top_k);
  if (p < 0 || p > t) return nullptr;
  return reinterpret_cast<const T*>(a.win) + (sq * a.w_cap + p % a.w_cap) * a.D;
}

}  // namespace

// Number of row splits per query row (workgroups sharing one query's rows).
static int attn_splits(int64_t rows, int top_k, int window, int H, int D, int dt) {
  if (!(dt == kBF16 && H == kAH && D == kAD)) return 1;
  const int64_t tiles = ceil_div(int64_t(top_k) + window, kTile);
  if (rows >= 256 || tiles <= 1) return 1;
  int64_t want = 256 / rows;
  if (want > tiles) want = tiles;
  if (want > 256) want = 256;
  return int(want < 1 ? 1 : want);
}

size_t attn_ws_bytes(int64_t rows, int H, int D, int top_k, int window, int dt) {
  const int ns = attn_splits(rows, top_k, window, H, D, dt);
  if (ns <= 1) return 0;
  return size_t(rows) * ns * H * (D + 2) * 4;
}

__global__ __launch_bounds__(256) void attn_mfma_kernel(AttnArgs a, int nsplit, int tiles_per_split) {
  __shared__ __attribute__((aligned(16))) unsigned char kvs[kTile * kKvRow];
  __shared__ __attribute__((aligned(16))) unsigned char vts[kAD * kVtRow];
  __shared__ int rowok[kTile];

  const int64_t r = blockIdx.y;
  const int split = blockIdx.x;
  const int64_t sq = r / a.n_q;
  const int64_t t = a.q_pos[r];
  const int nrows = a.top_k + a.window;
  const int64_t j0 = int64_t(split) * tiles_per_split * kTile;
  int64_t j1 = j0 + int64_t(tiles_per_split) * kTile;
  if (j1 > nrows) j1 = nrows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int head = 16 * wave + col;   // head of this lane in the score layout

  // Q^T as B operand: head `head`, dims ks*32 + g*8 .. +8
  bf16x8_t Qf[16];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + (r * kAH + head) * kAD + g * 8;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) Qf[ks] = *reinterpret_cast<const bf16x8_t*>(qp + ks * 32);
  }
  const float sl2 = a.scale * kLog2e;
  float m_run = neg_inf(), l_run = 0.f;
  f32x4_t O[32];
#pragma unroll
  for (int nt = 0; nt < 32; ++nt) O[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // gather assignment: thread -> row (tid & 31), 16-byte chunks (tid >> 5) + 8k, k < 8
  const int grow = tid & 31, gcb = tid >> 5;
  for (int64_t j = j0; j < j1; j += kTile) {
    const uint16_t* src = row_ptr<uint16_t>(a, r, sq, t, j + grow, int(j1));
    if (gcb == 0) rowok[grow] = src != nullptr;
    // all 8 loads issued back to back (a missing row reads the query row and is zeroed)
    const uint16_t* srcc = src ? src : reinterpret_cast<const uint16_t*>(a.q) + r * kAH * kAD;
    bf16x8_t vv8[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      vv8[k] = *reinterpret_cast<const bf16x8_t*>(srcc + (gcb + 8 * k) * 8);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = gcb + 8 * k;
      const bf16x8_t v = src ? vv8[k] : bf16x8_t{};
      *reinterpret_cast<bf16x8_t*>(&kvs[grow * kKvRow + c * 16]) = v;
      const uint16_t* hv = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint16_t*>(&vts[(c * 8 + e) * kVtRow + grow * 2]) = hv[e];
    }
    __syncthreads();

    // S^T: rows (4g+i) and (16+4g+i) against head `head`
    f32x4_t S0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, S1 = S0;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const bf16x8_t A0 = *reinterpret_cast<const bf16x8_t*>(&kvs[col * kKvRow + ks * 64 + g * 16]);
      const bf16x8_t A1 = *reinterpret_cast<const bf16x8_t*>(&kvs[(16 + col) * kKvRow + ks * 64 + g * 16]);
      S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, Qf[ks], S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, Qf[ks], S1, 0, 0, 0);
    }
    float s[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = rowok[4 * g + i] ? S0[i] * sl2 : neg_inf();
      s[4 + i] = rowok[16 + 4 * g + i] ? S1[i] * sl2 : neg_inf();
    }
    float tmax = s[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, s[i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == neg_inf()) ? 1.f : exp2f(m_run - m_new);
    float p[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = (s[i] == neg_inf()) ? 0.f : exp2f(s[i] - m_new);
      psum += p[i];
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // P as the A operand: row = head `col`, K slots (g, i) <-> rows {4g..4g+3, 16+4g..16+4g+3}
    bf16x8_t Pf;
#pragma unroll
    for (int i = 0; i < 8; ++i) Pf[i] = (__bf16)p[i];
    // output rows are heads 4g+i of this wave: fetch their rescale factors
    float ai[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) O[nt][i] *= ai[i];
      const unsigned char* vp = &vts[(nt * 16 + col) * kVtRow];
      const uint2 lo = *reinterpret_cast<const uint2*>(vp + 8 * g);
      const uint2 hi = *reinterpret_cast<const uint2*>(vp + 32 + 8 * g);
      bf16x8_t Vf;
      const uint4 vv = make_uint4(lo.x, lo.y, hi.x, hi.y);
      Vf = *reinterpret_cast<const bf16x8_t*>(&vv);
      O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Pf, Vf, O[nt], 0, 0, 0);
    }
    __syncthreads();
  }

  if (nsplit == 1) {
    const float zs = a.sink ? a.sink[head] * kLog2e : neg_inf();
    const float M = fmaxf(m_run, zs);
    float f = 0.f;
    if (M != neg_inf()) {
      const float em = (m_run == neg_inf()) ? 0.f : exp2f(m_run - M);
      const float den = l_run * em + ((zs == neg_inf()) ? 0.f : exp2f(zs - M));
      f = den > 0.f ? em / den : 0.f;
    }
    float fi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fi[i] = __shfl(f, 4 * g + i);
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + (r * kAH + 16 * wave) * kAD;
#pragma unroll
    for (int nt = 0; nt < 32; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        op[(4 * g + i) * kAD + nt * 16 + col] = f32_to_bf16(O[nt][i] * fi[i]);
  } else {
    // partial: [row][split][head][D + 2] = unnormalised O, then (max, sum) in base 2
    float* pp = reinterpret_cast<float*>(a.ws) + ((r * nsplit + split) * kAH + 16 * wave) * (kAD + 2);
#pragma unroll
    for (int nt = 0; nt < 32; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) pp[(4 * g + i) * (kAD + 2) + nt * 16 + col] = O[nt][i];
    if (g == 0) {
      pp[col * (kAD + 2) + kAD] = m_run;
      pp[col * (kAD + 2) + kAD + 1] = l_run;
    }
  }
}

// Merge the row splits of each (row, head) in split order: grid (H, rows). The split
// weights e^{m_s - M} / den are computed once into LDS; every output element then sums its
// nsplit partials with independent loads.
constexpr int kMaxSplit = 256;

template <typename T>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, int nsplit) {
  __shared__ float wgt[kMaxSplit];
  __shared__ float red[2][4];
  const int64_t r = blockIdx.y;
  const int h = blockIdx.x;
  const int H = a.H, D = a.D;
  const float* part = reinterpret_cast<const float*>(a.ws) + ((r * nsplit) * H + h) * (D + 2);
  const int64_t sstride = int64_t(H) * (D + 2);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float mi = neg_inf(), li = 0.f;
  if (tid < nsplit) {
    mi = part[tid * sstride + D];
    li = part[tid * sstride + D + 1];
  }
  const float zs = a.sink ? a.sink[h] * kLog2e : neg_inf();
  float M = wave_max(mi);
  if (lane == 0) red[0][wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3])), zs);
  const float e = (mi == neg_inf() || M == neg_inf()) ? 0.f : exp2f(mi - M);
  float den = wave_sum(li * e);
  if (lane == 0) red[1][wave] = den;
  __syncthreads();
  den = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  if (zs != neg_inf() && M != neg_inf()) den += exp2f(zs - M);
  if (tid < nsplit) wgt[tid] = den > 0.f ? e / den : 0.f;
  __syncthreads();
  T* op = reinterpret_cast<T*>(a.out) + (r * H + h) * D;
  for (int d = tid; d < D; d += blockDim.x) {
    float acc = 0.f;
    int sp = 0;
    for (; sp + 4 <= nsplit; sp += 4) {
      const float v0 = part[(sp + 0) * sstride + d], v1 = part[(sp + 1) * sstride + d];
      const float v2 = part[(sp + 2) * sstride + d], v3 = part[(sp + 3) * sstride + d];
      acc = fmaf(v0, wgt[sp + 0], acc);
      acc = fmaf(v1, wgt[sp + 1], acc);
      acc = fmaf(v2, wgt[sp + 2], acc);
      acc = fmaf(v3, wgt[sp + 3], acc);
    }
    for (; sp < nsplit; ++sp) acc = fmaf(part[sp * sstride + d], wgt[sp], acc);
    Elt<T>::store1(op + d, acc);
  }
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
  hipLaunchKernelGGL(attn_mfma_kernel, grid, dim3(256), 0, s, a, ns, tps);
  if (ns > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 g2(static_cast<unsigned>(a.H), static_cast<unsigned>(rows));
    hipLaunchKernelGGL(attn_combine_kernel<uint16_t>, g2, dim3(256), 0, s, a, ns);
  }
  return hipGetLastError();
}

}  // namespace csa
