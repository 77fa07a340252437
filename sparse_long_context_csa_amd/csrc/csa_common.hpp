// Device-side helpers shared by the libcsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---- bf16 <-> f32 (bf16 is the upper half of an fp32 bit pattern) -----------------------
__device__ __forceinline__ float bf16_lo(uint32_t two) { return __uint_as_float(two << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t two) { return __uint_as_float(two & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// f rounded to the nearest bf16 value (ties to even), as a float
__device__ __forceinline__ float round_to_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// cos and sin of the RoPE angle p * base^(-2j/rope_dim) (p may be negative): formed and reduced
// to [-pi, pi] in double precision, since positions reach millions of radians
__device__ __forceinline__ void rope_cos_sin(double p, int j, int rope_dim, double log2_base,
                                             float& c, float& s) {
  constexpr double kTwoPi = 6.283185307179586476925286766559;
  const double ang = p * exp2(-2.0 * double(j) / double(rope_dim) * log2_base);
  sincosf(float(ang - kTwoPi * rint(ang / kTwoPi)), &s, &c);
}

// x0, x1: channels 2j and 2j+1 held by adjacent lanes (this lane holds x, its DPP neighbour in
// [1,0,3,2] order the other one); returns this lane's rotated value
__device__ __forceinline__ float rope_pair_lane(float x, bool odd, float c, float s) {
  const float other = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xb1, 0xf, 0xf, false));
  return odd ? other * s + x * c : x * c - other * s;
}

// Storage-type traits: load/store 8 consecutive elements as fp32.
template <typename T> struct Elt;
template <> struct Elt<float> {
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static void load8(const float* p, float* o) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
  __device__ __forceinline__ static void store8(float* p, const float* v) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
  __device__ __forceinline__ static float load1(const float* p) { return *p; }
  __device__ __forceinline__ static void store1(float* p, float v) { *p = v; }
  __device__ __forceinline__ static float round(float v) { return v; }
};
template <> struct Elt<uint16_t> {   // bfloat16 storage
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static void load8(const uint16_t* p, float* o) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    o[0] = bf16_lo(a.x); o[1] = bf16_hi(a.x); o[2] = bf16_lo(a.y); o[3] = bf16_hi(a.y);
    o[4] = bf16_lo(a.z); o[5] = bf16_hi(a.z); o[6] = bf16_lo(a.w); o[7] = bf16_hi(a.w);
  }
  __device__ __forceinline__ static void store8(uint16_t* p, const float* v) {
    uint4 a;
    a.x = uint32_t(f32_to_bf16(v[0])) | (uint32_t(f32_to_bf16(v[1])) << 16);
    a.y = uint32_t(f32_to_bf16(v[2])) | (uint32_t(f32_to_bf16(v[3])) << 16);
    a.z = uint32_t(f32_to_bf16(v[4])) | (uint32_t(f32_to_bf16(v[5])) << 16);
    a.w = uint32_t(f32_to_bf16(v[6])) | (uint32_t(f32_to_bf16(v[7])) << 16);
    *reinterpret_cast<uint4*>(p) = a;
  }
  __device__ __forceinline__ static float load1(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store1(uint16_t* p, float v) { *p = f32_to_bf16(v); }
  __device__ __forceinline__ static float round(float v) { return round_to_bf16(v); }
};

// ---- causal visibility of compressed entries --------------------------------------------
// Entry i covers positions [m*i, m*(i+1)); a query at t may read it iff m*(i+1)-1 <= t.
__device__ __forceinline__ int64_t visible_entries(int64_t t, int m, int64_t cap) {
  if (t < 0) return 0;
  int64_t n = (t + 1) / m;
  return n < cap ? n : cap;
}

// ---- order-preserving key of an fp32 score ----------------------------------------------
// Larger score <=> larger key; -0 and +0 share a key.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ---- wave-level reductions --------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// popcount of the ballot bits of lanes below this one
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

}  // namespace csa
