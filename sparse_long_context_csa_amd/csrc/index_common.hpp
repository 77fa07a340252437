// Shared pieces of the lightning-indexer scans (index_scan.hip, index_prefill.hip): the
// MFMA operand layouts of the query and gates, the head-sum and maximum helpers.
//
// "DeepSeek V4-Flash: The Cost of Deciding What to Read", section "The Lightning Indexer":
// I(t,s) = sum_h w(t,h) * ReLU(q_I(t,h) . k_I(s)) over 64 indexer heads of dim 128.
#pragma once

#include <hip/hip_ext.h>

#include "csa_common.hpp"
#include "launch.hpp"

namespace csa {
namespace {

constexpr int kIH = 64;    // indexer heads on the MFMA paths
constexpr int kID = 128;   // indexer dim on the MFMA paths

// (the row's position already loaded: t = q_pos[r])
__device__ __forceinline__ int64_t row_visible_at(const ScanArgs& a, int64_t r, int64_t t) {
  const int64_t sq = r / a.n_q;
  int64_t cap = a.e_cap;
  if (a.e_count) {
    const int64_t ec = a.e_count[sq];
    cap = ec < cap ? (ec < 0 ? 0 : ec) : cap;
  }
  return visible_entries(t, a.m, cap);
}
__device__ __forceinline__ int64_t row_visible(const ScanArgs& a, int64_t r) {
  return row_visible_at(a, r, a.q_pos[r]);
}

// A operand of one query: heads 16*mt + (lane&15), channels ks*32 + g*8 .. +8 (g = lane>>4).
// The same channel order is used for the keys (B operand), so that in one load instruction
// the four lanes of a key read 64 contiguous bytes of its row.
__device__ __forceinline__ void load_query_A(const uint16_t* q, int lane, bf16x8_t (&A)[4][4]) {
  const int g = lane >> 4, col = lane & 15;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const uint16_t* p = q + (16 * mt + col) * kID + g * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) A[mt][ks] = *reinterpret_cast<const bf16x8_t*>(p + ks * 32);
  }
}

// gates of the heads held by this lane in the accumulator layout: 16*mt + 4*g + i
__device__ __forceinline__ void load_gates(const float* w, int lane, float (&wv)[4][4]) {
  const int g = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const float4 v = *reinterpret_cast<const float4*>(w + 16 * mt + 4 * g);
    wv[mt][0] = v.x; wv[mt][1] = v.y; wv[mt][2] = v.z; wv[mt][3] = v.w;
  }
}

// x[l] + x[l ^ 16] + x[l ^ 32] + x[l ^ 48] on every lane, with the gfx950 row swaps
// (v_permlane16_swap exchanges the odd 16-lane rows of one operand with the even rows of the
// other, v_permlane32_swap the upper half of one with the lower half of the other): a VALU
// exchange instead of LDS permutes. Each step adds a lane's value and its partner's, in
// either order (the same sum).
__device__ __forceinline__ float sum_rows4(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// max(x, 0) as a signed-integer max of the bit pattern: non-negative floats keep their bits,
// negative ones (-0 included) become +0. One integer instruction (a float max would first
// quiet each operand in IEEE mode).
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(__builtin_elementwise_max(__float_as_int(x), 0));
}

// order_key without folding -0 onto +0: a -0 maps just below +0. For maxima that feed a lower
// bound this is harmless (a maximum can only come out lower).
__device__ __forceinline__ uint32_t order_key_nz(float s) {
  const uint32_t u = __float_as_uint(s);
  return u ^ (uint32_t(int32_t(u) >> 31) | 0x80000000u);
}

// maximum over the 16 lanes of this lane's row (lanes 16j .. 16j+15 hold one key tile):
// integer maxima of order-preserving keys under rotations within the row (DPP row_ror), no
// LDS traffic; -0 comes back as +0
__device__ __forceinline__ uint32_t max16_key(uint32_t k) {
  k = __builtin_elementwise_max(k, uint32_t(__builtin_amdgcn_update_dpp(0, int(k), 0x121, 0xf, 0xf, false)));
  k = __builtin_elementwise_max(k, uint32_t(__builtin_amdgcn_update_dpp(0, int(k), 0x122, 0xf, 0xf, false)));
  k = __builtin_elementwise_max(k, uint32_t(__builtin_amdgcn_update_dpp(0, int(k), 0x124, 0xf, 0xf, false)));
  k = __builtin_elementwise_max(k, uint32_t(__builtin_amdgcn_update_dpp(0, int(k), 0x128, 0xf, 0xf, false)));
  return k;
}

// The 16 MFMAs of one 16-key group: acc[mt] = q[16 heads of mt] x the group's keys.
__device__ __forceinline__ void tile_mfma(const bf16x8_t (&A)[4][4], const bf16x8_t (&B)[4],
                                          f32x4_t (&acc)[4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][ks], B[ks], acc[mt], 0, 0, 0);
  }
}

// Gated ReLU sum over the lane's 16 heads (heads 16 mt + 4 g + i of key col), in two chains.
__device__ __forceinline__ float lane_part(const f32x4_t (&acc)[4], const float (&wv)[4][4]) {
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; mt += 2)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p0 = fmaf(wv[mt][i], relu_bits(acc[mt][i]), p0);
      p1 = fmaf(wv[mt + 1][i], relu_bits(acc[mt + 1][i]), p1);
    }
  return p0 + p1;
}

// Head sums of four 16-key groups at once from the lanes' partial sums x0..x3 (each over
// the lane's 16 heads; the 4 rows of the wave hold the 4 head quarters): a row-half swap
// adds rows g and g + 2 of two groups into one register (lanes 0-31 one group, 32-63 the
// other), a row swap then adds rows g and g + 1. Row 0 ends with group 0, row 1 with group
// 2, row 2 with group 1, row 3 with group 3: six instructions for 64 scores.
__device__ __forceinline__ float sum_groups4(float x0, float x1, float x2, float x3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0), __float_as_uint(x1),
                                                  false, false);
  const float s01 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x2), __float_as_uint(x3),
                                                  false, false);
  const float s23 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(s01), __float_as_uint(s23),
                                                  false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

constexpr int kBlk = 1024 + 64;   // LDS bytes per 4-key block of an LDS-DMA tile

// hipLaunchKernelGGL, or hipExtLaunchKernelGGL when the caller wants the dispatch's own
// start and stop events.
template <typename... KArgs, typename... Args>
static void launch_k(void (*kernel)(KArgs...), dim3 g, dim3 b, size_t shm, hipStream_t s,
                     hipEvent_t e0, hipEvent_t e1, Args... args) {
  if (e0 != nullptr && e1 != nullptr)
    hipExtLaunchKernelGGL(kernel, g, b, uint32_t(shm), s, e0, e1, 0u, KArgs(args)...);
  else
    hipLaunchKernelGGL(kernel, g, b, shm, s, KArgs(args)...);
}

}  // namespace
}  // namespace csa
