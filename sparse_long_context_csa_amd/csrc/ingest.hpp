// Decode-step ingest of one new token per sequence: the new rows go into the compressor
// tails and the window rings, and when the token completes an entry's m positions the
// entry is pooled into the caches ("DeepSeek V4-Flash: The Cost of Deciding What to Read",
// section "The compressor has two streams and they overlap": per-channel softmax pooling
// with a positional bias). Shared by the ingest kernel and the decode scan, which folds the
// same work into its own launch.
#pragma once

#include "csa_common.hpp"
#include "launch.hpp"

namespace csa {

// Pool 8 channels over n rows: fetch(j, a, x) gives row j's logits with the positional bias
// added (a[8]) and, when x is non-null, its values (x[8]). For n <= kRegM every row is fetched
// up front (one round trip to memory); longer pools take two passes (logits only for the
// maximum, then both). kRegs = false keeps to the two-pass form for every n (few registers:
// for callers that must not raise their own register budget).
constexpr int kRegM = 8;

template <bool kRegs, typename Fetch>
__device__ __forceinline__ void pool8_rows(int n, Fetch&& fetch, float* out) {
  if (kRegs && n <= kRegM) {
    float a[kRegM][8], xv[kRegM][8];
#pragma unroll
    for (int j = 0; j < kRegM; ++j)
      if (j < n) fetch(j, a[j], xv[j]);
    float mx[8], sum[8], acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) { mx[c] = a[0][c]; sum[c] = 0.f; acc[c] = 0.f; }
#pragma unroll
    for (int j = 1; j < kRegM; ++j)
      if (j < n)
#pragma unroll
        for (int c = 0; c < 8; ++c) mx[c] = fmaxf(mx[c], a[j][c]);
#pragma unroll
    for (int j = 0; j < kRegM; ++j)
      if (j < n)
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
  float mx[8], a[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) mx[c] = neg_inf();
  for (int j = 0; j < n; ++j) {
    fetch(j, a, nullptr);
#pragma unroll
    for (int c = 0; c < 8; ++c) mx[c] = fmaxf(mx[c], a[c]);
  }
  float sum[8], acc[8], xv[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) { sum[c] = 0.f; acc[c] = 0.f; }
  for (int j = 0; j < n; ++j) {
    fetch(j, a, xv);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float e = expf(a[c] - mx[c]);
      sum[c] += e;
      acc[c] = fmaf(e, xv[c], acc[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) out[c] = acc[c] / sum[c];
}

// Row j (< m) of one stream's block: its x/z from memory (x0 + j*stride), except row `own`
// whose values are passed in registers (xo, zo); the bias row b0 + j*bstride added to z. Row
// `own` is loaded too (its memory slot is stale) and then replaced by a select, so that no
// branch splits the loads of the rows: they all go out before the first one is waited for.
template <typename T>
__device__ __forceinline__ void fetch_row8(const T* x0, const T* z0, int64_t stride,
                                           const T* b0, int bstride, int j, int own,
                                           const float* xo, const float* zo, float* a,
                                           float* x) {
  const bool o = j == own;
  Elt<T>::load8(z0 + j * stride, a);
  if (x != nullptr) Elt<T>::load8(x0 + j * stride, x);
  float bb[8];
  Elt<T>::load8(b0 + j * bstride, bb);
#pragma unroll
  for (int c = 0; c < 8; ++c) a[c] = (o ? zo[c] : a[c]) + bb[c];
  if (x != nullptr)
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = o ? xo[c] : x[c];
}

// Pool 8 channels over the m rows of one stream's block (csa_compress's entry).
template <typename T, bool kRegs = true>
__device__ __forceinline__ void pool8(const T* x0, const T* z0, int64_t stride, const T* b0,
                                      int bstride, int m, int own, const float* xo,
                                      const float* zo, float* out) {
  pool8_rows<kRegs>(
      m,
      [&](int j, float* a, float* x) {
        fetch_row8<T>(x0, z0, stride, b0, bstride, j, own, xo, zo, a, x);
      },
      out);
}

// The overlapped two-stream entry (csa_compress_c4a's): one softmax over the m a rows of the
// entry's own block (x0/z0, row `own` in registers, bias b0) and the m b rows of the block
// before (xb0/zb0, bias bb0; none when xb0 is null: a sequence's first entry).
template <typename T, bool kRegs = true>
__device__ __forceinline__ void pool8_c4a(const T* x0, const T* z0, const T* xb0, const T* zb0,
                                          int64_t stride, const T* b0, const T* bb0, int m,
                                          int own, const float* xo, const float* zo,
                                          float* out) {
  pool8_rows<kRegs>(
      xb0 != nullptr ? 2 * m : m,
      [&](int j, float* a, float* x) {
        if (j < m) fetch_row8<T>(x0, z0, stride, b0, stride, j, own, xo, zo, a, x);
        else fetch_row8<T>(xb0, zb0, stride, bb0, stride, j - m, -1, xo, zo, a, x);
      },
      out);
}

// Vectors of 8 channels one sequence's ingest covers: main stream, rings, indexer stream.
__device__ __forceinline__ int ingest_vectors(const IngestArgs& a) {
  return (a.dim >> 3) + a.n_ring * (a.dim >> 3) + (a.idx_dim >> 3);
}

// The per-head RMSNorm (kv_gamma, eps 1e-6) and RoPE at position p on the last kv_rope_dim
// channels of a key/value row, 8 channels c0 .. c0 + 7 per lane; the row's 64 vectors are the
// 64 lanes of this wave (dim 512), which all call this together.
//   ["DeepSeek V4-Flash: The Cost of Deciding What to Read", "Key and value are the same
//   vector": RMSNorm per head on the KV head, RoPE on the last 64 dimensions, so that every
//   key/value row carries its position's rotation; vLLM fuses KV RoPE with the window-key
//   insertion ("Two cache hierarchies, and lcm(4, 128)").]
template <typename T>
__device__ __forceinline__ void prep_kv_row8(const IngestArgs& a, int64_t p, int c0, int d,
                                             float* res) {
  if (a.kv_gamma != nullptr) {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) ss = fmaf(res[k], res[k], ss);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    const float scale = 1.f / sqrtf(ss / float(d) + 1e-6f);
    float g[8];
    Elt<T>::load8(static_cast<const T*>(a.kv_gamma) + c0, g);
#pragma unroll
    for (int k = 0; k < 8; ++k) res[k] = res[k] * scale * g[k];
  }
  const int r0 = d - a.kv_rope_dim;
  if (a.kv_rope_dim > 0) {   // uniform
    // lane j forms the angle of pair j once; the lanes holding the rotated channels fetch
    // theirs by shuffles
    const int lane = threadIdx.x & 63;
    float cs_l = 1.f, sn_l = 0.f;
    if (lane < a.kv_rope_dim / 2)
      rope_cos_sin(double(p), lane, a.kv_rope_dim, a.rope_log2_base, cs_l, sn_l);
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
      const int j = (c0 + k - r0) >> 1;
      const float cs = __shfl(cs_l, j & 63), sn = __shfl(sn_l, j & 63);
      if (c0 + k >= r0) {
        const float x0 = res[k], x1 = res[k + 1];
        res[k] = x0 * cs - x1 * sn;
        res[k + 1] = x0 * sn + x1 * cs;
      }
    }
  }
}

// Vector v of sequence sq: [0, vd) main stream (tail row, pooled entry when complete), then
// n_ring * vd window-ring vectors (row t % w_cap of ring c from win_new[c], when given), then
// [vd + n_ring * vd, + vi) the indexer stream (tail row; pooled key when complete and
// pool_index). With dim 512 (vd = 64) the main row and every ring row are one wave each.
// The pooled entry and every new window row get the RMSNorm and RoPE at t of prep_kv_row8
// when kv_gamma or kv_rope_dim asks for them (dim 512 then).
template <typename T, bool kRegs = true>
__device__ __forceinline__ void ingest_vector(const IngestArgs& a, int64_t sq, int v,
                                              bool pool_index) {
  const int vd = a.dim >> 3, vr = a.n_ring * vd;
  const int64_t t = a.pos[sq];
  if (t < 0) return;
  const int m = a.m;
  const int slot = int(t % m);
  const bool complete = ((t + 1) % m) == 0;
  const int64_t e = (t + 1) / m - 1;
  const bool prep = a.kv_gamma != nullptr || a.kv_rope_dim > 0;
  if (v >= vd && v < vd + vr) {
    const int r = v - vd;
    const int c = r / vd;
    const int c0 = (r % vd) << 3;
    const T* src = (const T*)a.win_new[c];
    if (src == nullptr) return;   // uniform over the ring row's wave
    float w8[8];
    Elt<T>::load8(src + sq * a.dim + c0, w8);
    if (prep) prep_kv_row8<T>(a, t, c0, a.dim, w8);
    Elt<T>::store8((T*)a.win[c] + (sq * a.w_cap + t % a.w_cap) * a.dim + c0, w8);
    return;
  }
  const bool main = v < vd;
  const int d = main ? a.dim : a.idx_dim;
  const int c0 = (main ? v : v - vd - vr) << 3;
  const T* xn = (const T*)(main ? a.x_new : a.xi_new) + sq * d + c0;
  const T* zn = (const T*)(main ? a.z_new : a.zi_new) + sq * d + c0;
  T* xt = (T*)(main ? a.x_tail : a.xi_tail) + sq * m * d + c0;
  T* zt = (T*)(main ? a.z_tail : a.zi_tail) + sq * m * d + c0;
  // Every load (the new rows, the tail rows and biases the entry pools) goes out before the
  // first store: the tail slot and the b ring row this step writes are never read (the new row
  // is pooled from registers), so the loads make a single round trip to memory.
  float xo[8], zo[8];
  Elt<T>::load8(xn, xo);
  Elt<T>::load8(zn, zo);
  // the overlapped main compressor's b stream: the new row goes to the two-block ring (row
  // t % 2m); the entry reads the other block's half
  const bool c4a = main && a.xb_new != nullptr;
  float xb[8], zb[8];
  T* xr = nullptr;
  T* zr = nullptr;
  if (c4a) {
    Elt<T>::load8((const T*)a.xb_new + sq * d + c0, xb);
    Elt<T>::load8((const T*)a.zb_new + sq * d + c0, zb);
    xr = (T*)a.xb_tail + sq * 2 * m * d + c0;
    zr = (T*)a.zb_tail + sq * 2 * m * d + c0;
  }
  const bool pool = complete && e < a.e_cap && (main || pool_index);
  float res[8];
  if (pool) {
    if (c4a) {
      const int64_t h = int64_t((e - 1) & 1) * m * d;   // block e - 1 (none for entry 0)
      pool8_c4a<T, kRegs>(xt, zt, e > 0 ? xr + h : nullptr, e > 0 ? zr + h : nullptr, d,
                          (const T*)a.bias + c0, (const T*)a.bias_b + c0, m, slot, xo, zo, res);
    } else {
      pool8<T, kRegs>(xt, zt, d, (const T*)(main ? a.bias : a.bias_i) + c0, d, m, slot, xo,
                      zo, res);
    }
  }
  Elt<T>::store8(xt + slot * d, xo);
  Elt<T>::store8(zt + slot * d, zo);
  if (c4a) {
    const int rb = int(t % (2 * m));
    Elt<T>::store8(xr + rb * d, xb);
    Elt<T>::store8(zr + rb * d, zb);
  }
  if (pool) {
    // the entry's RMSNorm and RoPE at t (the newest position it pools): its 64 vectors are
    // this wave's 64 lanes
    if (main && prep) prep_kv_row8<T>(a, t, c0, d, res);
    if (main && a.kv_fmt == kKvFp8) {   // the pooled entry in T (bf16), then the FP8 form
      store_fp8_entry8(static_cast<uint8_t*>(a.kv) + (sq * a.e_cap + e) * kFp8EntryBytes, c0,
                       res, true);
    } else if (main && a.kv_fmt == kKvFp4) {   // the same for the FP4 form (the whole wave)
#pragma unroll
      for (int k = 0; k < 8; ++k) res[k] = round_to_bf16(res[k]);
      store_fp4_entry8(static_cast<uint8_t*>(a.kv) + (sq * a.e_cap + e) * kFp4EntryBytes, c0,
                       res);
    } else {
      T* dst = (T*)(main ? a.kv : a.k_idx) + (sq * a.e_cap + e) * d + c0;
      Elt<T>::store8(dst, res);
    }
  }
}

// Query preparation of sequence sq for every attention call (IngestArgs::n_qprep), share `part`
// of `parts` workgroups: one wave per (call, head) vector (lane l: channels 8 l .. 8 l + 7,
// q_dim <= 512), kB vectors loaded together: the per-head
// RMSNorm (eps 1e-6) when the call has a gamma, then RoPE at +pos on the last q_rope_dim
// channels, stored once in the storage dtype. The row's pair angles (q_rope_dim <= 64) are
// formed once per wave, lane l taking pair l & 31, and fetched by shuffles.
template <typename T>
__device__ __forceinline__ void prep_queries(const IngestArgs& a, int64_t sq, int part,
                                             int parts) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int64_t t = a.pos[sq];
  float cs_l = 1.f, sn_l = 0.f;
  if (a.q_rope_dim > 0 && (lane & 31) < a.q_rope_dim / 2)
    rope_cos_sin(double(t), lane & 31, a.q_rope_dim, a.rope_log2_base, cs_l, sn_l);
  const int c0 = lane * 8, r0 = a.q_dim - a.q_rope_dim;
  const bool live = c0 < a.q_dim;
  constexpr int kB = 2;
  const int n_jobs = a.n_qprep * a.q_heads;
  for (int j0 = (part * nw + wave) * kB; j0 < n_jobs; j0 += parts * nw * kB) {
    float v[kB][8];
#pragma unroll
    for (int i = 0; i < kB; ++i) {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[i][k] = 0.f;
      const int job = j0 + i;
      if (job < n_jobs && live) {
        const int c = job / a.q_heads, h = job % a.q_heads;
        Elt<T>::load8(static_cast<const T*>(a.qsrc[c]) + (sq * a.q_heads + h) * a.q_dim + c0,
                      v[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      const int job = j0 + i;
      if (job >= n_jobs) break;   // uniform
      const int c = job / a.q_heads, h = job % a.q_heads;
      if (a.qgamma[c] == nullptr && a.q_rope_dim == 0) continue;   // call c uses its own query
      if (a.qgamma[c] != nullptr) {   // uniform
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) ss = fmaf(v[i][k], v[i][k], ss);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
        const float scale = 1.f / sqrtf(ss / float(a.q_dim) + 1e-6f);
        float g[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (live) Elt<T>::load8(static_cast<const T*>(a.qgamma[c]) + c0, g);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[i][k] = v[i][k] * scale * g[k];
      }
      if (a.q_rope_dim > 0) {
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
          const int j = (c0 + k - r0) >> 1;
          const float cs = __shfl(cs_l, j & 31), sn = __shfl(sn_l, j & 31);
          if (live && c0 + k >= r0) {
            const float x0 = v[i][k], x1 = v[i][k + 1];
            v[i][k] = x0 * cs - x1 * sn;
            v[i][k + 1] = x0 * sn + x1 * cs;
          }
        }
      }
      if (live)
        Elt<T>::store8(static_cast<T*>(a.qdst[c]) + (sq * a.q_heads + h) * a.q_dim + c0, v[i]);
    }
  }
}

// The pooled indexer key vector v (8 channels) of the entry that position t completes,
// computed from the tails and the new row (the tail slot of t is not read).
template <typename T, bool kRegs = true>
__device__ __forceinline__ void pool_index_vector(const IngestArgs& a, int64_t sq, int64_t t,
                                                  int v, float* res) {
  const int m = a.m, d = a.idx_dim, c0 = v << 3;
  const int slot = int(t % m);
  float xo[8], zo[8];
  Elt<T>::load8((const T*)a.xi_new + sq * d + c0, xo);
  Elt<T>::load8((const T*)a.zi_new + sq * d + c0, zo);
  pool8<T, kRegs>((const T*)a.xi_tail + sq * m * d + c0, (const T*)a.zi_tail + sq * m * d + c0,
                  d, (const T*)a.bias_i + c0, d, m, slot, xo, zo, res);
}

}  // namespace csa
