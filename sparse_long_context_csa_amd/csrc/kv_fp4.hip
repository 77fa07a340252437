// FP4 storage of the main KV entries (288 bytes per 512-channel entry).
//
// "DeepSeek-V4.1-Flash's KV-Cache Compression, Checked Down to the Byte", section 4 (Cell 3
// "FP4 range analysis"): E2M1 elements, one E4M3 scale per 16 channels, no second-level global
// scale. The "DeepSeek-V4.1-Flash" interactive study, "FP4 main KV": the full latent is
// quantised after RoPE and attention dequantises the cached values before using them.
//
// quantize_kv_fp4_kernel: one wave per entry, lane l holding channels 8 l .. 8 l + 7; the lane
// pair of a 16-channel block agrees on its scale by a shuffle (store_fp4_entry8).
// dequantize_kv_fp4_kernel: thread per 8 channels into bf16 (exact: element x scale is a bf16
// value).
#include "csa_common.hpp"
#include "launch.hpp"

namespace csa {
namespace {

constexpr int kEntryDim = 512;

template <typename T>
__global__ __launch_bounds__(256) void quantize_kv_fp4_kernel(const T* __restrict__ x,
                                                              uint8_t* __restrict__ out,
                                                              int64_t n_vec) {
  // n_vec is a multiple of 64 and a wave's 64 vectors are one entry: a wave is either wholly
  // inside or wholly past the end, so the pair shuffle always has both lanes
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n_vec) return;
  const int64_t row = i >> 6;
  const int c0 = int(i & 63) * 8;
  float v[8];
  Elt<T>::load8(x + row * kEntryDim + c0, v);
  store_fp4_entry8(out + row * kFp4EntryBytes, c0, v);
}

__global__ __launch_bounds__(256) void dequantize_kv_fp4_kernel(const uint8_t* __restrict__ in,
                                                                uint16_t* __restrict__ out,
                                                                int64_t n_vec) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n_vec) return;
  const int64_t row = i >> 6;
  const int c = int(i & 63);
  const bf16x8_t b = fp4_entry_chunk8(in + row * kFp4EntryBytes, c);
  *reinterpret_cast<bf16x8_t*>(out + row * kEntryDim + 8 * c) = b;
}

}  // namespace

hipError_t launch_quantize_kv_fp4(int dt, const void* x, void* out, int64_t n_rows,
                                  hipStream_t s) {
  const int64_t n_vec = n_rows * (kEntryDim / 8);
  if (n_vec == 0) return hipSuccess;
  const dim3 grid(unsigned((n_vec + 255) / 256));
  if (dt == kBF16)
    hipLaunchKernelGGL(quantize_kv_fp4_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), static_cast<uint8_t*>(out), n_vec);
  else
    hipLaunchKernelGGL(quantize_kv_fp4_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(x), static_cast<uint8_t*>(out), n_vec);
  return hipGetLastError();
}

hipError_t launch_dequantize_kv_fp4(const void* in, void* out, int64_t n_rows, hipStream_t s) {
  const int64_t n_vec = n_rows * (kEntryDim / 8);
  if (n_vec == 0) return hipSuccess;
  const dim3 grid(unsigned((n_vec + 255) / 256));
  hipLaunchKernelGGL(dequantize_kv_fp4_kernel, grid, dim3(256), 0, s,
                     static_cast<const uint8_t*>(in), static_cast<uint16_t*>(out), n_vec);
  return hipGetLastError();
}

}  // namespace csa
