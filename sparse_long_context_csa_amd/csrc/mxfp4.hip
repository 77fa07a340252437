// MXFP4 quantisation of rows (indexer keys): E2M1 codes and E8M0 block scales (mxfp4.hpp).
//
// Four threads per block of 32 channels, 8 channels each: the block maximum by two quad
// exchanges (DPP), each thread writes its 4 code bytes, the first of the four the scale byte.
#include "csa_common.hpp"
#include "launch.hpp"
#include "mxfp4.hpp"

namespace csa {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(const T* __restrict__ x,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales,
                                                             int64_t n_groups) {
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;   // 8-channel group
  const bool live = t < n_groups;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (live) Elt<T>::load8(x + t * 8, v);
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
  // the 4 threads of a block are lanes 4k .. 4k+3 of the wave (n_groups is a multiple of 4)
  am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(am), 0xb1, 0xf, 0xf, false)));
  am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(am), 0x4e, 0xf, 0xf, false)));
  const int s = mx_shared_exp(am);
  if (!live) return;
  uint32_t packed = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) packed |= e2m1_code(ldexpf(v[i], -s)) << (4 * i);
  reinterpret_cast<uint32_t*>(codes)[t] = packed;
  if ((t & 3) == 0) scales[t >> 2] = uint8_t(s + 127);
}

}  // namespace

hipError_t launch_quantize_mxfp4(int dt, const void* x, void* codes, void* scales, int64_t n_rows,
                                 int dim, hipStream_t s) {
  const int64_t groups = n_rows * (dim / 8);
  if (groups == 0) return hipSuccess;
  const unsigned grid = unsigned((groups + 255) / 256);
  if (dt == kBF16)
    hipLaunchKernelGGL(quantize_mxfp4_kernel<uint16_t>, dim3(grid), dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), static_cast<uint8_t*>(codes),
                       static_cast<uint8_t*>(scales), groups);
  else
    hipLaunchKernelGGL(quantize_mxfp4_kernel<float>, dim3(grid), dim3(256), 0, s,
                       static_cast<const float*>(x), static_cast<uint8_t*>(codes),
                       static_cast<uint8_t*>(scales), groups);
  return hipGetLastError();
}

}  // namespace csa
