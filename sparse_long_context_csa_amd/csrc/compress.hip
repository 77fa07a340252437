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
