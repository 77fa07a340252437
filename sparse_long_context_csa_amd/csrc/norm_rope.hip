// Per-head RMSNorm and partial RoPE in one pass (the elementwise work around the attention).
//
// "DeepSeek V4-Flash: The Cost of Deciding What to Read", section "Key and value are the same
// vector": RMSNorm per head on the queries and on the single head of the compressed KV entries
// just before the core attention; RoPE on the last 64 dimensions of each head, and on the
// output with position -i, which undoes the rotation the shared key/value carried in.
//
// One wave per (row, head) vector of up to 512 channels at a time; lane l owns channels
// 8 l .. 8 l + 7 (one 16-byte load and store for bf16). The mean square is a wave sum (DPP row
// rotations, then the row swaps). RoPE pairs (2j, 2j+1) of the rotated part never straddle
// lanes; the angle pos * base^(-2j/rope_dim) is formed and reduced in double precision
// (positions reach millions of radians), once per row, then the rotation runs in fp32.
#include <math.h>

#include "csa_common.hpp"
#include "launch.hpp"

namespace csa {

namespace {

__device__ __forceinline__ float wave_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// One workgroup per row: the row's rope_dim / 2 rotation angles are formed once (double
// precision, reduced to [-pi, pi], then fp32 sine and cosine) into LDS and shared by its heads;
// wave w takes heads w, w + 4, ... (one vector per iteration, lane l channels 8 l .. 8 l + 7).
constexpr int kMaxPairs = 256;   // rope_dim <= 512
template <typename T>
__global__ __launch_bounds__(256) void norm_rope_kernel(const T* __restrict__ x,
                                                        const T* __restrict__ gamma,
                                                        const int64_t* __restrict__ pos,
                                                        T* out, int n_heads, int dim,
                                                        int rope_dim, double log2_base,
                                                        float eps, int flags) {
  __shared__ float cs[kMaxPairs], sn[kMaxPairs];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;
  const bool rope = (flags & 2) != 0;
  if (rope) {
    const double p = double(pos[row]) * ((flags & 4) ? -1.0 : 1.0);
    constexpr double kTwoPi = 6.283185307179586476925286766559;
    for (int j = threadIdx.x; j < rope_dim / 2; j += 256) {
      const double ang = p * exp2(-2.0 * double(j) / double(rope_dim) * log2_base);
      const float red = float(ang - kTwoPi * rint(ang / kTwoPi));   // in [-pi, pi]
      float s_, c_;
      sincosf(red, &s_, &c_);
      cs[j] = c_;
      sn[j] = s_;
    }
    __syncthreads();
  }
  const int c0 = lane * 8;
  const bool live = c0 < dim;
  const int r0 = dim - rope_dim;
  float g[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
  if ((flags & 1) && live) Elt<T>::load8(gamma + c0, g);
  for (int h = wave; h < n_heads; h += 4) {
    const int64_t vec = row * n_heads + h;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (live) Elt<T>::load8(x + vec * dim + c0, v);
    if (flags & 1) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) ss = fmaf(v[c], v[c], ss);
      const float scale = 1.f / sqrtf(wave_sum(ss) / float(dim) + eps);
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = v[c] * scale * g[c];
    }
    if (rope && live && c0 + 8 > r0) {
#pragma unroll
      for (int c = 0; c < 8; c += 2) {
        const int ch = c0 + c;
        if (ch >= r0) {
          const int j = (ch - r0) >> 1;
          const float a = v[c], b = v[c + 1];
          v[c] = a * cs[j] - b * sn[j];
          v[c + 1] = a * sn[j] + b * cs[j];
        }
      }
    }
    if (live) Elt<T>::store8(out + vec * dim + c0, v);
  }
}

}  // namespace

hipError_t launch_norm_rope(int dt, const void* x, const void* gamma, const int64_t* pos,
                            void* out, int64_t n_rows, int n_heads, int dim, int rope_dim,
                            float base, float eps, int flags, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(n_rows)), block(256);
  const double lb = log2(double(base));
  if (dt == kBF16)
    hipLaunchKernelGGL(norm_rope_kernel<uint16_t>, grid, block, 0, s, (const uint16_t*)x,
                       (const uint16_t*)gamma, pos, (uint16_t*)out, n_heads, dim, rope_dim, lb,
                       eps, flags);
  else
    hipLaunchKernelGGL(norm_rope_kernel<float>, grid, block, 0, s, (const float*)x,
                       (const float*)gamma, pos, (float*)out, n_heads, dim, rope_dim, lb, eps,
                       flags);
  return hipGetLastError();
}

}  // namespace csa
