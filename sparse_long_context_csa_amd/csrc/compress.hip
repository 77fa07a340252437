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
#include "launch.hpp"

namespace csa {

// Pool 8 channels over m rows. Row j's x/z come from memory (x0 + j*stride) except row
// `own` whose values are passed in registers (xo, zo). For m <= kRegM every row is loaded
// up front (one round trip to memory); longer entries take two passes over the logits.
constexpr int kRegM = 8;

template <typename T>
__device__ __forceinline__ void pool8(const T* x0, const T* z0, int64_t stride, const T* b0,
                                      int bstride, int m, int own, const float* xo,
                                      const float* zo, float* out) {
  if (m <= kRegM) {
    float a[kRegM][8], xv[kRegM][8];
#pragma unroll
    for (int j = 0; j < kRegM; ++j) {
      if (j < m) {
        float bb[8];
        if (j == own) {
#pragma unroll
          for (int c = 0; c < 8; ++c) { a[j][c] = zo[c]; xv[j][c] = xo[c]; }
        } else {
          Elt<T>::load8(z0 + j * stride, a[j]);
          Elt<T>::load8(x0 + j * stride, xv[j]);
        }
        Elt<T>::load8(b0 + j * bstride, bb);
#pragma unroll
        for (int c = 0; c < 8; ++c) a[j][c] += bb[c];
      }
    }
    float mx[8], sum[8], acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) { mx[c] = a[0][c]; sum[c] = 0.f; acc[c] = 0.f; }
#pragma unroll
    for (int j = 1; j < kRegM; ++j)
      if (j < m)
#pragma unroll
        for (int c = 0; c < 8; ++c) mx[c] = fmaxf(mx[c], a[j][c]);
#pragma unroll
    for (int j = 0; j < kRegM; ++j)
      if (j < m)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float e = expf(a[j][c] - mx[c]);
          sum[c] += e;
          acc[c] = fmaf(e, xv[j][c], acc[c]);
        }
#pragma unroll
    for (int c = 0; c < 8; ++c) out[c] = acc[c] / sum[c];
    return;
  }
  float mx[8], a[8], bb[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) mx[c] = neg_inf();
  for (int j = 0; j < m; ++j) {
    if (j == own) {
#pragma unroll
      for (int c = 0; c < 8; ++c) a[c] = zo[c];
    } else {
      Elt<T>::load8(z0 + j * stride, a);
    }
    Elt<T>::load8(b0 + j * bstride, bb);
#pragma unroll
    for (int c = 0; c < 8; ++c) mx[c] = fmaxf(mx[c], a[c] + bb[c]);
  }
  float sum[8], acc[8], xv[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) { sum[c] = 0.f; acc[c] = 0.f; }
  for (int j = 0; j < m; ++j) {
    if (j == own) {
#pragma unroll
      for (int c = 0; c < 8; ++c) { a[c] = zo[c]; xv[c] = xo[c]; }
    } else {
      Elt<T>::load8(z0 + j * stride, a);
      Elt<T>::load8(x0 + j * stride, xv);
    }
    Elt<T>::load8(b0 + j * bstride, bb);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float e = expf(a[c] + bb[c] - mx[c]);
      sum[c] += e;
      acc[c] = fmaf(e, xv[c], acc[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) out[c] = acc[c] / sum[c];
}

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

hipError_t launch_compress(int dt, const void* x, const void* z, const void* bias, void* out,
                           int64_t n_seq, int64_t n_tok, int64_t out_seq_stride, int dim, int m,
                           hipStream_t s) {
  const int64_t n_ent = n_tok / m;
  const int64_t total = n_seq * n_ent * (dim / 8);
  if (total == 0) return hipSuccess;
  const int64_t stride = out_seq_stride ? out_seq_stride : n_ent * dim;
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

// ---- decode ingest: new rows -> tails / rings, pool the block when it completes ---------
// One thread per 8-channel vector: vectors [0, vd) main stream, [vd, vd+vi) indexer stream,
// then n_ring * vd window-ring vectors. blockIdx.y = sequence.
template <typename T>
__global__ __launch_bounds__(256) void ingest_kernel(IngestArgs a) {
  const int64_t sq = blockIdx.y;
  const int vd = a.dim >> 3, vi = a.idx_dim >> 3;
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t = a.pos[sq];
  if (t < 0) return;
  const int m = a.m;
  const int slot = int(t % m);
  const bool complete = ((t + 1) % m) == 0;
  const int64_t e = (t + 1) / m - 1;
  if (tid < vd + vi) {
    const bool main = tid < vd;
    const int d = main ? a.dim : a.idx_dim;
    const int c0 = (main ? tid : tid - vd) << 3;
    const T* xn = (const T*)(main ? a.x_new : a.xi_new) + sq * d + c0;
    const T* zn = (const T*)(main ? a.z_new : a.zi_new) + sq * d + c0;
    T* xt = (T*)(main ? a.x_tail : a.xi_tail) + sq * m * d + c0;
    T* zt = (T*)(main ? a.z_tail : a.zi_tail) + sq * m * d + c0;
    float xo[8], zo[8];
    Elt<T>::load8(xn, xo);
    Elt<T>::load8(zn, zo);
    Elt<T>::store8(xt + slot * d, xo);
    Elt<T>::store8(zt + slot * d, zo);
    if (complete && e < a.e_cap) {
      float res[8];
      pool8<T>(xt, zt, d, (const T*)(main ? a.bias : a.bias_i) + c0, d, m, slot, xo, zo, res);
      T* dst = (T*)(main ? a.kv : a.k_idx) + (sq * a.e_cap + e) * d + c0;
      Elt<T>::store8(dst, res);
    }
    return;
  }
  const int r = tid - vd - vi;
  if (r >= a.n_ring * vd) return;
  const int c = r / vd;
  const int c0 = (r % vd) << 3;
  const T* src = (const T*)a.win_new[c];
  if (src == nullptr) return;
  float v[8];
  Elt<T>::load8(src + sq * a.dim + c0, v);
  Elt<T>::store8((T*)a.win[c] + (sq * a.w_cap + t % a.w_cap) * a.dim + c0, v);
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
