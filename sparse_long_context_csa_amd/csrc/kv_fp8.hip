// FP8 storage of the main KV entries.
//
// "DeepSeek V4-Flash: The Cost of Deciding What to Read", "What the cache costs, checked
// four ways": a shared key/value entry of head dimension 512 keeps its 64 rotary dimensions in
// bf16 and the other 448 in FP8, 576 bytes. Element format: OCP E4M3 (no scale: the 576 bytes
// leave no room for one, and the entries are RMS-normalised per head).
//
// quantize_kv_fp8_kernel: thread per 8 channels (64 per entry); channels below 448 become eight
// E4M3 codes (one 8-byte store), the rest eight bf16 values (one 16-byte store).
// dequantize_kv_fp8_kernel: the inverse into bf16 (exact: every E4M3 value is a bf16 value).
#include "csa_common.hpp"
#include "launch.hpp"

namespace csa {
namespace {

constexpr int kEntryDim = 512;

template <typename T>
__global__ __launch_bounds__(256) void quantize_kv_fp8_kernel(const T* __restrict__ x,
                                                              uint8_t* __restrict__ out,
                                                              int64_t n_vec) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n_vec) return;
  const int64_t row = i >> 6;
  const int c0 = int(i & 63) * 8;
  float v[8];
  Elt<T>::load8(x + row * kEntryDim + c0, v);
  store_fp8_entry8(out + row * kFp8EntryBytes, c0, v, false);
}

__global__ __launch_bounds__(256) void dequantize_kv_fp8_kernel(const uint8_t* __restrict__ in,
                                                                uint16_t* __restrict__ out,
                                                                int64_t n_vec) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n_vec) return;
  const int64_t row = i >> 6;
  const int c0 = int(i & 63) * 8;
  const uint8_t* e = in + row * kFp8EntryBytes;
  uint4 r;
  if (c0 < kFp8Nope) {
    const uint2 w = *reinterpret_cast<const uint2*>(e + c0);
    const bf16x8_t b = e4m3x8_to_bf16(w.x, w.y);
    r = *reinterpret_cast<const uint4*>(&b);
  } else {
    r = *reinterpret_cast<const uint4*>(e + kFp8Nope + 2 * (c0 - kFp8Nope));
  }
  *reinterpret_cast<uint4*>(out + row * kEntryDim + c0) = r;
}

}  // namespace

hipError_t launch_quantize_kv_fp8(int dt, const void* x, void* out, int64_t n_rows,
                                  hipStream_t s) {
  const int64_t n_vec = n_rows * (kEntryDim / 8);
  if (n_vec == 0) return hipSuccess;
  const dim3 grid(unsigned((n_vec + 255) / 256));
  if (dt == kBF16)
    hipLaunchKernelGGL(quantize_kv_fp8_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), static_cast<uint8_t*>(out), n_vec);
  else
    hipLaunchKernelGGL(quantize_kv_fp8_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(x), static_cast<uint8_t*>(out), n_vec);
  return hipGetLastError();
}

hipError_t launch_dequantize_kv_fp8(const void* in, void* out, int64_t n_rows, hipStream_t s) {
  const int64_t n_vec = n_rows * (kEntryDim / 8);
  if (n_vec == 0) return hipSuccess;
  const dim3 grid(unsigned((n_vec + 255) / 256));
  hipLaunchKernelGGL(dequantize_kv_fp8_kernel, grid, dim3(256), 0, s,
                     static_cast<const uint8_t*>(in), static_cast<uint16_t*>(out), n_vec);
  return hipGetLastError();
}

}  // namespace csa
