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

// Number of row splits per query row (workgroups sharing one query's rows): few query rows
// (decode) spread each row list over up to 256 workgroups in all, one tile or more each:
// a wave's chain of LDS reads and MFMAs per tile is latency-bound, so tiles run in
// parallel workgroups and the partial results are merged afterwards.
constexpr int kMinTilesPerSplit = 1;
static int attn_splits(int64_t rows, int top_k, int window, int H, int D, int dt) {
  if (!(dt == kBF16 && H == kAH && D == kAD)) return 1;
  const int64_t tiles = ceil_div(int64_t(top_k) + window, kTile);
  if (rows >= 256 || tiles < 2) return 1;
  int64_t want = ceil_div(tiles, kMinTilesPerSplit);
  const int64_t cap = 256 / rows;
  if (want > cap) want = cap;
  return int(want < 1 ? 1 : want);
}

// Partials of split s of row r: the unnormalised output in the MFMA accumulator layout,
// [wave][nt][lane] float4 (64 heads x 512 dims), then (max, sum) per head in base 2.
constexpr int64_t kPartO = int64_t(kAH) * kAD;   // floats per (row, split)

size_t attn_ws_bytes(int64_t rows, int H, int D, int top_k, int window, int dt) {
  const int ns = attn_splits(rows, top_k, window, H, D, dt);
  if (ns <= 1) return 0;
  return size_t(rows) * ns * (kPartO + 2 * kAH) * 4;
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

  // gather assignment: thread -> rows 4*ra .. 4*ra+3 (ra = tid & 7), 16-byte chunks cp and
  // cp + 32 (cp = tid >> 3); rows past the list read the query row and are zeroed
  const int ra = tid & 7, cp = tid >> 3;
  const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + r * kAH * kAD;
  bf16x8_t vv[4][2];
  bool okr[4];
  const uint16_t* srcs[4];
  auto locate = [&](int64_t j) {   // row pointers of tile j (the ids load here)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      srcs[i] = row_ptr<uint16_t>(a, r, sq, t, j + 4 * ra + i, int(j1));
      okr[i] = srcs[i] != nullptr;
    }
  };
  auto gather = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t* sc = okr[i] ? srcs[i] : qrow;
      vv[i][0] = *reinterpret_cast<const bf16x8_t*>(sc + cp * 8);
      vv[i][1] = *reinterpret_cast<const bf16x8_t*>(sc + (cp + 32) * 8);
    }
  };
  if (j0 < j1) locate(j0);
  // Q^T as B operand: head `head`, dims ks*32 + g*8 .. +8 (loads while the ids arrive)
  bf16x8_t Qf[16];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + (r * kAH + head) * kAD + g * 8;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) Qf[ks] = *reinterpret_cast<const bf16x8_t*>(qp + ks * 32);
  }
  if (j0 < j1) gather();
  const float sl2 = a.scale * kLog2e;
  float m_run = neg_inf(), l_run = 0.f;
  f32x4_t O[32];
#pragma unroll
  for (int nt = 0; nt < 32; ++nt) O[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int64_t j = j0; j < j1; j += kTile) {
    // tile j to LDS: row-major (A operand of S^T) and transposed, 4 rows per 8-byte store
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!okr[i]) { vv[i][0] = bf16x8_t{}; vv[i][1] = bf16x8_t{}; }
      if (cp == 0) rowok[4 * ra + i] = okr[i];
      *reinterpret_cast<bf16x8_t*>(&kvs[(4 * ra + i) * kKvRow + cp * 16]) = vv[i][0];
      *reinterpret_cast<bf16x8_t*>(&kvs[(4 * ra + i) * kKvRow + (cp + 32) * 16]) = vv[i][1];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = cp + 32 * h;
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vv[0][h]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vv[1][h]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vv[2][h]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vv[3][h]);
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        // dims 2*e2 (low halves) and 2*e2+1 (high halves) of the 4 rows
        const uint32_t lo01 = __builtin_amdgcn_perm(w1[e2], w0[e2], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(w3[e2], w2[e2], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(w1[e2], w0[e2], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(w3[e2], w2[e2], 0x07060302u);
        *reinterpret_cast<uint2*>(&vts[(c * 8 + 2 * e2) * kVtRow + ra * 8]) = make_uint2(lo01, lo23);
        *reinterpret_cast<uint2*>(&vts[(c * 8 + 2 * e2 + 1) * kVtRow + ra * 8]) = make_uint2(hi01, hi23);
      }
    }
    __syncthreads();
    // the next tile's rows load while this one computes
    if (j + kTile < j1) {
      locate(j + kTile);
      gather();
    }

    // S^T: rows (4g+i) and (16+4g+i) against head `head`
    // four independent accumulator chains (even / odd K steps of both 16-row halves)
    f32x4_t S0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, S1 = S0, S2 = S0, S3 = S0;
#pragma unroll
    for (int ks = 0; ks < 16; ks += 2) {
      const bf16x8_t A0 = *reinterpret_cast<const bf16x8_t*>(&kvs[col * kKvRow + ks * 64 + g * 16]);
      const bf16x8_t A1 = *reinterpret_cast<const bf16x8_t*>(&kvs[(16 + col) * kKvRow + ks * 64 + g * 16]);
      const bf16x8_t A2 = *reinterpret_cast<const bf16x8_t*>(&kvs[col * kKvRow + ks * 64 + 64 + g * 16]);
      const bf16x8_t A3 = *reinterpret_cast<const bf16x8_t*>(&kvs[(16 + col) * kKvRow + ks * 64 + 64 + g * 16]);
      S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, Qf[ks], S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, Qf[ks], S1, 0, 0, 0);
      S2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A2, Qf[ks + 1], S2, 0, 0, 0);
      S3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A3, Qf[ks + 1], S3, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) { S0[i] += S2[i]; S1[i] += S3[i]; }
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
      const uint4 vv4 = make_uint4(lo.x, lo.y, hi.x, hi.y);
      Vf = *reinterpret_cast<const bf16x8_t*>(&vv4);
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
    // partial in the accumulator layout (16-byte stores), then (max, sum) per head
    const int64_t rs = r * nsplit + split;
    f32x4_t* pp = reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(a.ws) + rs * kPartO) +
                  wave * 32 * kWave + lane;
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) pp[nt * kWave] = O[nt];
    if (g == 0) {
      float2* ml = reinterpret_cast<float2*>(reinterpret_cast<float*>(a.ws) +
                                             int64_t(gridDim.y) * nsplit * kPartO) + rs * kAH;
      ml[head] = make_float2(m_run, l_run);
    }
  }
}

// Merge the row splits in split order. Grid (32, rows): workgroup x covers the heads of
// accumulator wave w = x / 8 and the dims of 4 accumulator columns; its first 16 threads
// compute the split weights e^{m_s - M} / den of those 16 heads into LDS, then every thread
// sums its float4 (4 heads, 1 dim) over the splits with independent loads.
constexpr int kMaxSplit = 256;

__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, int nsplit) {
  __shared__ float wgt[kMaxSplit][16];
  __shared__ float2 mls[kMaxSplit][16];
  const int64_t r = blockIdx.y;
  const int w = blockIdx.x >> 3;
  const int nt = (blockIdx.x & 7) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t rows = gridDim.y;
  const float* base = reinterpret_cast<const float*>(a.ws);
  const float2* ml = reinterpret_cast<const float2*>(base + rows * nsplit * kPartO) +
                     r * nsplit * kAH;
  const f32x4_t* part = reinterpret_cast<const f32x4_t*>(base + r * nsplit * kPartO) +
                        (w * 32 + nt) * kWave + lane;
  constexpr int64_t sstride = kPartO / 4;   // float4 per split
  // the first kSplitRegs partials load first, together with the (max, sum) pairs
  constexpr int kSplitRegs = 32;
  f32x4_t v[kSplitRegs];
#pragma unroll
  for (int sp = 0; sp < kSplitRegs; ++sp)
    v[sp] = sp < nsplit ? part[sp * sstride] : f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int q = threadIdx.x; q < nsplit * 16; q += blockDim.x)
    mls[q >> 4][q & 15] = ml[(q >> 4) * kAH + 16 * w + (q & 15)];
  __syncthreads();
  if (threadIdx.x < 16) {
    const int h = 16 * w + threadIdx.x;
    const float zs = a.sink ? a.sink[h] * kLog2e : neg_inf();
    float M = zs;
    for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, mls[sp][threadIdx.x].x);
    float den = (zs == neg_inf() || M == neg_inf()) ? 0.f : exp2f(zs - M);
    for (int sp = 0; sp < nsplit; ++sp) {
      const float2 m2 = mls[sp][threadIdx.x];
      const float e = (m2.x == neg_inf() || M == neg_inf()) ? 0.f : exp2f(m2.x - M);
      wgt[sp][threadIdx.x] = e;
      den += m2.y * e;
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    for (int sp = 0; sp < nsplit; ++sp) wgt[sp][threadIdx.x] *= inv;
  }
  __syncthreads();
  const int g = lane >> 4, col = lane & 15;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < kSplitRegs; ++sp)
    if (sp < nsplit)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(v[sp][i], wgt[sp][4 * g + i], acc[i]);
  for (int sp = kSplitRegs; sp < nsplit; ++sp) {
    const f32x4_t x = part[sp * sstride];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(x[i], wgt[sp][4 * g + i], acc[i]);
  }
  uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + (r * kAH + 16 * w + 4 * g) * kAD + nt * 16 + col;
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
    const dim3 g2(32u, static_cast<unsigned>(rows));
    hipLaunchKernelGGL(attn_combine_kernel, g2, dim3(256), 0, s, a, ns);
  }
  return hipGetLastError();
}

}  // namespace csa
