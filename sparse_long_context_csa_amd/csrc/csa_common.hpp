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

// Round to nearest even (the gfx950 conversion instruction); NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// f rounded to the nearest bf16 value (ties to even), as a float
__device__ __forceinline__ float round_to_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// ---- FP8 main-cache entries --------------------------------------------------------------
// "DeepSeek V4-Flash: The Cost of Deciding What to Read", "What the cache costs, checked
// four ways": a 512-dim key/value entry keeps its 64 rotary dims in bf16 and the rest in FP8,
// 576 bytes. Channels 0 .. 447 are OCP E4M3 codes (bias 7, largest finite 448, no infinity),
// channels 448 .. 511 follow as bf16.
constexpr int kFp8Nope = 448;          // E4M3 channels of an entry
constexpr int kFp8EntryBytes = 576;    // 448 + 2 * 64

// E4M3 code of x: nearest value, ties to the even code, magnitudes past 448 to 448, a zero
// magnitude as +0. The grid spacing at |x| is 2^(e-3), e = floor(log2 |x|) clamped below at
// -6 (the subnormal spacing 2^-9); scaling by powers of two keeps every step exact.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const float a = fabsf(x);
  const int e = int(__float_as_uint(fmaxf(a, 0x1p-6f)) >> 23) - 127;
  const float inv_ulp = __uint_as_float(uint32_t(127 + 3 - e) << 23);   // 2^(3-e)
  const float ulp = __uint_as_float(uint32_t(127 - 3 + e) << 23);       // 2^(e-3)
  const float q = fminf(rintf(a * inv_ulp) * ulp, 448.f);
  uint32_t code;
  if (q >= 0x1p-6f) {
    const uint32_t qb = __float_as_uint(q);
    code = ((((qb >> 23) & 0xffu) - 127u + 7u) << 3) | ((qb >> 20) & 7u);
  } else {
    code = uint32_t(q * 512.f);   // subnormal m * 2^-9, m = 0 .. 7
  }
  return (x < 0.f && q > 0.f) ? (code | 0x80u) : code;
}

// Eight E4M3 codes (two dwords, code i in byte i) -> eight bf16 values, exact (every E4M3
// value is a bf16 value): gfx950 v_cvt_scalef32_pk_bf16_fp8 with scale 1.
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Channels c0 .. c0+7 (c0 % 8 == 0) of an FP8 entry from fp32 values v, stored as E4M3
// (c0 < 448) or bf16. via_bf16: each value is first rounded to bf16 (the entry as a bf16 cache
// would hold it), so that both parts quantise the same stored value.
__device__ __forceinline__ void store_fp8_entry8(uint8_t* entry, int c0, const float* v,
                                                 bool via_bf16) {
  if (c0 < kFp8Nope) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i >> 2] |= e4m3_code(via_bf16 ? round_to_bf16(v[i]) : v[i]) << (8 * (i & 3));
    *reinterpret_cast<uint2*>(entry + c0) = make_uint2(w[0], w[1]);
  } else {
    uint4 b;
    b.x = uint32_t(f32_to_bf16(v[0])) | (uint32_t(f32_to_bf16(v[1])) << 16);
    b.y = uint32_t(f32_to_bf16(v[2])) | (uint32_t(f32_to_bf16(v[3])) << 16);
    b.z = uint32_t(f32_to_bf16(v[4])) | (uint32_t(f32_to_bf16(v[5])) << 16);
    b.w = uint32_t(f32_to_bf16(v[6])) | (uint32_t(f32_to_bf16(v[7])) << 16);
    *reinterpret_cast<uint4*>(entry + kFp8Nope + 2 * (c0 - kFp8Nope)) = b;
  }
}

// ---- FP4 main-cache entries --------------------------------------------------------------
// "DeepSeek-V4.1-Flash's KV-Cache Compression, Checked Down to the Byte", section 4 (Cell 3):
// the whole 512-channel entry as E2M1 elements with one E4M3 scale per 16 channels and no
// global scale, 512 / 2 + 512 / 16 = 288 bytes. Bytes 0 .. 255: element codes, channel 2i in
// the low nibble of byte i; bytes 256 .. 287: the scale codes, byte 256 + g for channels
// 16 g .. 16 g + 15. Block scale: the E4M3 value nearest to max|x| / 6 (the block maximum on
// E2M1's largest magnitude); elements: nearest magnitude times the scale, ties to the even code.
constexpr int kFp4CodeBytes = 256;
constexpr int kFp4EntryBytes = 288;

// value of a non-negative E4M3 code (0 .. 0x7e): m 2^-9 when the exponent field is 0
__device__ __forceinline__ float e4m3_pos_value(uint32_t code) {
  const uint32_t e = code >> 3, m = code & 7u;
  return e == 0u ? float(m) * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// E2M1 code of x under a block scale s > 0: the nearest of the magnitudes {0, .5, 1, 1.5, 2, 3,
// 4, 6} times s, ties to the even code, past 6 s to 6 s; a zero magnitude is code 0. The
// decision points are the midpoints times s, exact in fp32 (at most 7 significant bits, never
// below 2^-11), so every comparison is exact.
__device__ __forceinline__ uint32_t e2m1_code_scaled(float x, float s) {
  const float a = fabsf(x);
  // midpoints reached (those below an even code) or passed (the others): no branches
  const uint32_t c = uint32_t(a > 0.25f * s) + uint32_t(a >= 0.75f * s) +
                     uint32_t(a > 1.25f * s) + uint32_t(a >= 1.75f * s) +
                     uint32_t(a > 2.5f * s) + uint32_t(a >= 3.5f * s) + uint32_t(a > 5.f * s);
  return c | (uint32_t(x < 0.f && c != 0u) << 3);
}

// Channels c0 .. c0+7 (c0 % 8 == 0) of an FP4 entry from their stored values v: the lane
// pair (c0 / 8 even, odd) shares a 16-channel block and its scale; every lane of the wave must
// call this together (the pair exchanges its maxima by a shuffle). amax / 6 is correctly
// rounded in fp32, and since amax carries at most 24 significant bits it never lands on, or
// crosses, an E4M3 rounding midpoint it does not equal, so e4m3_code rounds it as the exact
// quotient would be rounded.
__device__ __forceinline__ void store_fp4_entry8(uint8_t* entry, int c0, const float* v) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  const uint32_t sc = e4m3_code(amax / 6.f);
  const float s = e4m3_pos_value(sc);
  uint32_t w = 0u;
  if (sc != 0u) {
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= e2m1_code_scaled(v[i], s) << (4 * i);
  }
  *reinterpret_cast<uint32_t*>(entry + (c0 >> 1)) = w;
  if (((c0 >> 3) & 1) == 0) entry[kFp4CodeBytes + (c0 >> 4)] = uint8_t(sc);
}

// Eight FP4 element codes (one dword, channel k of the eight in nibble k) times the block
// scale s -> eight bf16 values, exact: v_cvt_scalef32_pk_f32_fp4 with scale 1 (the scaled
// conversions of gfx950 apply only the exponent of their fp32 scale, so the E4M3 scale is a
// separate multiply), then v_cvt_pk_bf16_f32 (the product is a bf16 value).
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t w, float s) {
  const auto f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const auto f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const auto f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const auto f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  bf16x8_t r;
  r[0] = (__bf16)(f0[0] * s); r[1] = (__bf16)(f0[1] * s);
  r[2] = (__bf16)(f1[0] * s); r[3] = (__bf16)(f1[1] * s);
  r[4] = (__bf16)(f2[0] * s); r[5] = (__bf16)(f2[1] * s);
  r[6] = (__bf16)(f3[0] * s); r[7] = (__bf16)(f3[1] * s);
  return r;
}

// the two block scales of a chunk pair: E4M3 codes in the low two bytes of sc2 -> fp32, exact
__device__ __forceinline__ void e4m3x2_scales(uint32_t sc2, float& s0, float& s1) {
  const auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sc2, 1.0f, false);
  s0 = f[0];
  s1 = f[1];
}

// chunk c (channels 8c .. 8c+7) of an FP4 entry as bf16
__device__ __forceinline__ bf16x8_t fp4_entry_chunk8(const uint8_t* e, int c) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(e + 4 * c);
  return fp4x8_to_bf16(w, e4m3_pos_value(e[kFp4CodeBytes + (c >> 1)]));
}

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
