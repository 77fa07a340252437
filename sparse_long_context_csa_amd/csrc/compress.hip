// Compressor: learned channel-wise softmax pooling of m consecutive rows into one entry.
//
// "DeepSeek V4-Flash: The Cost of Deciding What to Read", section "The compressor has two
// streams and they overlap": the weights are per channel, a softmax over the pooled
// positions runs independently for each channel and the entry is the weighted sum of the
// rows; the CSA/HCA layer tables give each stream a learnable positional bias of shape
// m x d (added to the logits by position within the entry). "DeepSeek-V4.1-Flash" study,
// "CSA2: separate producing, selecting, and reading": groups pooled without overlap.
//
// HBM-bound streaming kernel: each thread owns 8 consecutive channels of one entry and
// reads them with 16-byte (bf16) or 2 x 16-byte (fp32) loads, so a wave covers 512
// contiguous channels of a row; m <= 16 rows are pooled in registers (two passes over the
// logits: max, then exp-weighted sum), fp32 arithmetic, one rounded store.
#include "csa_common.hpp"
#include "ingest.hpp"
#include "launch.hpp"

namespace csa {

template <typename T>
__global__ __launch_bounds__(256) void compress_kernel(const T* __restrict__ x,
                                                       const T* __restrict__ z,
                                                       const T* __restrict__ bias,
                                                       T* __restrict__ out, int64_t n_seq,
                                                       int64_t n_ent, int64_t out_seq_stride,
                                                       int dim, int m) {
  const int vpe = dim >> 3;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= n_seq * n_ent * vpe) return;
  const int v = int(gid % vpe);
  const int64_t se = gid / vpe;
  const int64_t e = se % n_ent, sq = se / n_ent;
  const int c0 = v << 3;
  const int64_t row0 = (sq * n_ent + e) * m;
  float res[8];
  pool8<T>(x + row0 * dim + c0, z + row0 * dim + c0, dim, bias + c0, dim, m, -1, nullptr,
           nullptr, res);
  Elt<T>::store8(out + sq * out_seq_stride + e * dim + c0, res);
}

// Long entries (m > 16, HCA's m' = 128): a workgroup pools one entry for 8 vectors (64
// channels) with 32 row groups -- thread (group g, vector v) takes rows g, g + 32, ... < m
// (4 at most), all of them and their biases loaded in one round before any arithmetic, and
// keeps a partial softmax (maximum, sum, weighted sum) over them. The 8 groups of a wave merge
// by lane shuffles (the lanes of one vector are 8 apart), the 4 waves through LDS. Every
// input row is read once.
constexpr int kWideGroups = 32;
constexpr int kWideVecs = 8;
constexpr int kWideRows = 4;   // rows per thread: m <= kWideGroups * kWideRows = 128

// (m, s, a) of two partial softmaxes over disjoint rows, merged (an empty one has m = -inf)
__device__ __forceinline__ void merge_softmax(float& m, float& s, float& a, float mo, float so,
                                              float ao) {
  const float mn = fmaxf(m, mo);
  if (mn == neg_inf()) return;
  const float e = m == neg_inf() ? 0.f : expf(m - mn);
  const float eo = mo == neg_inf() ? 0.f : expf(mo - mn);
  s = s * e + so * eo;
  a = a * e + ao * eo;
  m = mn;
}

template <typename T>
__global__ __launch_bounds__(256) void compress_wide_kernel(const T* __restrict__ x,
                                                            const T* __restrict__ z,
                                                            const T* __restrict__ bias,
                                                            T* __restrict__ out, int64_t n_ent,
                                                            int64_t out_seq_stride, int dim,
                                                            int m) {
  __shared__ float part[3][4][kWideVecs][8];
  const int vl = threadIdx.x % kWideVecs, grp = threadIdx.x / kWideVecs;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nvb = (dim / 8 + kWideVecs - 1) / kWideVecs;   // channel blocks per entry
  const int64_t bid = blockIdx.x;
  const int v = int(bid % nvb) * kWideVecs + vl;
  const int64_t e = (bid / nvb) % n_ent, sq = bid / nvb / n_ent;
  const bool live = v * 8 < dim;
  const int c0 = v * 8;
  const int64_t row0 = (sq * n_ent + e) * m;
  float mx[8], sum[8], acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) { mx[c] = neg_inf(); sum[c] = 0.f; acc[c] = 0.f; }
  if (live) {
    float xv[kWideRows][8], lv[kWideRows][8], bv[kWideRows][8];
#pragma unroll
    for (int i = 0; i < kWideRows; ++i) {
      const int j = grp + i * kWideGroups;
      if (j < m) {
        Elt<T>::load8(x + (row0 + j) * dim + c0, xv[i]);
        Elt<T>::load8(z + (row0 + j) * dim + c0, lv[i]);
        Elt<T>::load8(bias + j * dim + c0, bv[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < kWideRows; ++i) {
      if (grp + i * kWideGroups < m) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          lv[i][c] += bv[i][c];
          mx[c] = fmaxf(mx[c], lv[i][c]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kWideRows; ++i) {
      if (grp + i * kWideGroups < m) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float pw = expf(lv[i][c] - mx[c]);
          sum[c] += pw;
          acc[c] = fmaf(pw, xv[i][c], acc[c]);
        }
      }
    }
  }
  // the wave's 8 groups of this vector: lanes vl, vl + 8, ..., vl + 56
#pragma unroll
  for (int o = 8; o < 64; o <<= 1) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float mo = __shfl_xor(mx[c], o), so = __shfl_xor(sum[c], o), ao = __shfl_xor(acc[c], o);
      merge_softmax(mx[c], sum[c], acc[c], mo, so, ao);
    }
  }
  if (lane < kWideVecs) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      part[0][wave][vl][c] = mx[c];
      part[1][wave][vl][c] = sum[c];
      part[2][wave][vl][c] = acc[c];
    }
  }
  __syncthreads();
  // thread (vector vl, channel c) of the first 64 merges the 4 waves in order
  if (threadIdx.x < kWideVecs * 8) {
    const int vv = threadIdx.x >> 3, c = threadIdx.x & 7;
    const int v2 = int(bid % nvb) * kWideVecs + vv;
    if (v2 * 8 < dim) {
      float M = part[0][0][vv][c], S = part[1][0][vv][c], A = part[2][0][vv][c];
#pragma unroll
      for (int w2 = 1; w2 < 4; ++w2)
        merge_softmax(M, S, A, part[0][w2][vv][c], part[1][w2][vv][c], part[2][w2][vv][c]);
      Elt<T>::store1(out + sq * out_seq_stride + e * dim + v2 * 8 + c, A / S);
    }
  }
}

hipError_t launch_compress(int dt, const void* x, const void* z, const void* bias, void* out,
                           int64_t n_seq, int64_t n_tok, int64_t out_seq_stride, int dim, int m,
                           hipStream_t s) {
  const int64_t n_ent = n_tok / m;
  const int64_t total = n_seq * n_ent * (dim / 8);
  if (total == 0) return hipSuccess;
  const int64_t stride = out_seq_stride ? out_seq_stride : n_ent * dim;
  if (m > 16) {
    const dim3 gw(unsigned(int64_t((dim / 8 + kWideVecs - 1) / kWideVecs) * n_ent * n_seq));
    if (dt == kBF16)
      hipLaunchKernelGGL(compress_wide_kernel<uint16_t>, gw, dim3(256), 0, s,
                         (const uint16_t*)x, (const uint16_t*)z, (const uint16_t*)bias,
                         (uint16_t*)out, n_ent, stride, dim, m);
    else
      hipLaunchKernelGGL(compress_wide_kernel<float>, gw, dim3(256), 0, s, (const float*)x,
                         (const float*)z, (const float*)bias, (float*)out, n_ent, stride, dim,
                         m);
    return hipGetLastError();
  }
  const dim3 grid(unsigned((total + 255) / 256)), block(256);
  if (dt == kBF16)
    hipLaunchKernelGGL(compress_kernel<uint16_t>, grid, block, 0, s, (const uint16_t*)x,
                       (const uint16_t*)z, (const uint16_t*)bias, (uint16_t*)out, n_seq, n_ent,
                       stride, dim, m);
  else
    hipLaunchKernelGGL(compress_kernel<float>, grid, block, 0, s, (const float*)x,
                       (const float*)z, (const float*)bias, (float*)out, n_seq, n_ent, stride,
                       dim, m);
  return hipGetLastError();
}

// ---- overlapped two-stream compressor ("c4a" at m = 4) ----------------------------------
// Entry e of the chunk pools the a-stream rows of its own block [m e, m e + m) and the
// b-stream rows of the block before [m(e-1), m e) (for e = 0 the caller's previous rows, or
// none at the start of a sequence) under one softmax over the 2m logits per channel. Each
// thread owns 8 channels of one entry; the rows stream through an online softmax (a running
// maximum, the sum and the weighted sum rescaled when the maximum rises), so the registers do
// not grow with m. All 2m rows' loads of a thread are independent and issue together.
template <typename T>
__device__ __forceinline__ void c4a_row(const T* x, const T* z, const T* b, float (&mx)[8],
                                        float (&sum)[8], float (&acc)[8]) {
  float xv[8], zv[8], bv[8];
  Elt<T>::load8(x, xv);
  Elt<T>::load8(z, zv);
  Elt<T>::load8(b, bv);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float l = zv[c] + bv[c];
    if (l > mx[c]) {
      const float r = expf(mx[c] - l);        // 0 when mx is -inf (first row)
      sum[c] *= r;
      acc[c] *= r;
      mx[c] = l;
    }
    const float p = expf(l - mx[c]);
    sum[c] += p;
    acc[c] = fmaf(p, xv[c], acc[c]);
  }
}

// Rows of the entry: a-part (its block) then b-part (the block before, or the caller's
// previous rows for e = 0, or none at the start of a sequence).
template <typename T>
struct C4aRows {
  const T *xa, *za, *xb, *zb;
  bool has_b;
};
template <typename T>
__device__ __forceinline__ C4aRows<T> c4a_rows(const T* xa, const T* za, const T* xb,
                                               const T* zb, const T* xb_prev, const T* zb_prev,
                                               int64_t sq, int64_t e, int64_t n_tok, int m,
                                               int dim, int c0) {
  C4aRows<T> r;
  const int64_t ra = sq * n_tok + e * m;
  r.xa = xa + ra * dim + c0;
  r.za = za + ra * dim + c0;
  r.has_b = e > 0 || xb_prev != nullptr;
  const int64_t rb = e > 0 ? sq * n_tok + (e - 1) * m : sq * m;
  r.xb = (e > 0 ? xb : xb_prev) + rb * dim + c0;
  r.zb = (e > 0 ? zb : zb_prev) + rb * dim + c0;
  return r;
}

// kM > 0: m == kM rows per part, all 2 kM rows loaded before any arithmetic (one round trip),
// then a two-pass softmax in registers; kM == 0: any m, the online softmax above.
template <typename T, int kM>
__global__ __launch_bounds__(256) void compress_c4a_kernel(
    const T* __restrict__ xa, const T* __restrict__ za, const T* __restrict__ xb,
    const T* __restrict__ zb, const T* __restrict__ ba, const T* __restrict__ bb,
    const T* __restrict__ xb_prev, const T* __restrict__ zb_prev, T* __restrict__ out,
    int64_t n_seq, int64_t n_ent, int64_t out_seq_stride, int dim, int m) {
  const int vpe = dim >> 3;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= n_seq * n_ent * vpe) return;
  const int v = int(gid % vpe);
  const int64_t se = gid / vpe;
  const int64_t e = se % n_ent, sq = se / n_ent;
  const int c0 = v << 3;
  const C4aRows<T> R = c4a_rows(xa, za, xb, zb, xb_prev, zb_prev, sq, e, n_ent * m, m, dim, c0);
  float res[8];
  if constexpr (kM > 0) {
    float xv[2 * kM][8], lv[2 * kM][8];
#pragma unroll
    for (int j = 0; j < kM; ++j) {
      Elt<T>::load8(R.xa + j * dim, xv[j]);
      Elt<T>::load8(R.za + j * dim, lv[j]);
      if (R.has_b) {
        Elt<T>::load8(R.xb + j * dim, xv[kM + j]);
        Elt<T>::load8(R.zb + j * dim, lv[kM + j]);
      }
    }
    float mx[8], sum[8], acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) { mx[c] = neg_inf(); sum[c] = 0.f; acc[c] = 0.f; }
#pragma unroll
    for (int j = 0; j < 2 * kM; ++j) {
      if (j >= kM && !R.has_b) break;
      float bv[8];
      Elt<T>::load8((j < kM ? ba : bb) + (j % kM) * dim + c0, bv);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        lv[j][c] += bv[c];
        mx[c] = fmaxf(mx[c], lv[j][c]);
      }
    }
#pragma unroll
    for (int j = 0; j < 2 * kM; ++j) {
      if (j >= kM && !R.has_b) break;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float p = expf(lv[j][c] - mx[c]);
        sum[c] += p;
        acc[c] = fmaf(p, xv[j][c], acc[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) res[c] = acc[c] / sum[c];
  } else {
    float mx[8], sum[8], acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) { mx[c] = neg_inf(); sum[c] = 0.f; acc[c] = 0.f; }
#pragma unroll 4
    for (int j = 0; j < m; ++j)
      c4a_row<T>(R.xa + j * dim, R.za + j * dim, ba + j * dim + c0, mx, sum, acc);
    if (R.has_b) {
#pragma unroll 4
      for (int j = 0; j < m; ++j)
        c4a_row<T>(R.xb + j * dim, R.zb + j * dim, bb + j * dim + c0, mx, sum, acc);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) res[c] = acc[c] / sum[c];
  }
  Elt<T>::store8(out + sq * out_seq_stride + e * dim + c0, res);
}

hipError_t launch_compress_c4a(int dt, const void* xa, const void* za, const void* xb,
                               const void* zb, const void* ba, const void* bb,
                               const void* xb_prev, const void* zb_prev, void* out,
                               int64_t n_seq, int64_t n_tok, int64_t out_seq_stride, int dim,
                               int m, hipStream_t s) {
  const int64_t n_ent = n_tok / m;
  const int64_t total = n_seq * n_ent * (dim / 8);
  if (total == 0) return hipSuccess;
  const int64_t stride = out_seq_stride ? out_seq_stride : n_ent * dim;
  const dim3 grid(unsigned((total + 255) / 256)), block(256);
#define CSA_C4A(TT, KM)                                                                      \
  do {                                                                                       \
    auto* kfn = &compress_c4a_kernel<TT, KM>;                                                \
    hipLaunchKernelGGL(kfn, grid, block, 0, s, (const TT*)xa, (const TT*)za, (const TT*)xb, \
                       (const TT*)zb, (const TT*)ba, (const TT*)bb, (const TT*)xb_prev,      \
                       (const TT*)zb_prev, (TT*)out, n_seq, n_ent, stride, dim, m);          \
  } while (0)
  if (dt == kBF16) {
    if (m == 4) CSA_C4A(uint16_t, 4);
    else if (m == 2) CSA_C4A(uint16_t, 2);
    else if (m == 1) CSA_C4A(uint16_t, 1);
    else CSA_C4A(uint16_t, 0);
  } else {
    if (m == 4) CSA_C4A(float, 4);
    else if (m == 2) CSA_C4A(float, 2);
    else if (m == 1) CSA_C4A(float, 1);
    else CSA_C4A(float, 0);
  }
#undef CSA_C4A
  return hipGetLastError();
}

// ---- decode ingest: new rows -> tails / rings, pool the block when it completes ---------
// One thread per 8-channel vector (see ingest_vector). blockIdx.y = sequence.
template <typename T>
__global__ __launch_bounds__(256) void ingest_kernel(IngestArgs a) {
  const int64_t sq = blockIdx.y;
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v < ingest_vectors(a)) ingest_vector<T>(a, sq, v, true);
}

hipError_t launch_ingest(const IngestArgs& a, hipStream_t s) {
  const int vd = a.dim / 8, vi = a.idx_dim / 8;
  const int nthreads = vd + vi + a.n_ring * vd;
  const dim3 grid(unsigned((nthreads + 255) / 256), unsigned(a.n_seq)), block(256);
  if (a.dt == kBF16)
    hipLaunchKernelGGL(ingest_kernel<uint16_t>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(ingest_kernel<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace csa
