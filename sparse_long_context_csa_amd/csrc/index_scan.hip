// Lightning-indexer scan: I(t,s) = sum_h w(t,h) * ReLU(q_I(t,h) . K_s) for every candidate.
//
// "DeepSeek V4-Flash: The Cost of Deciding What to Read", section "The Lightning Indexer":
// 64 indexer heads of dim 128 per query, one compressed indexer key per entry, a rectified
// dot product per head, summed with the per-head gate w; section "The indexer is O(n), and
// that is the ceiling": the scan touches every visible entry and never becomes sparse.
//
// Kernels:
//  * scan_stream_kernel (bf16, 64 heads x 128, whole visible rows): few query rows, many keys
//    (decode). The contraction is a [64 heads x 128] x [128 x 16 keys] MFMA
//    (v_mfma_f32_16x16x32_bf16) per tile with the query in VGPRs as the A operand; key rows
//    move HBM -> LDS by global_load_lds_dwordx4 (1 KiB of consecutive memory per
//    instruction, no VGPRs held by loads in flight) through a ring of LDS slots per wave, and
//    each key row is read once. ReLU, gate and head sum run on the accumulator lanes; two
//    row swaps finish the head sum. For long rows an item (a chunk of positions) also leaves
//    its candidate segment for the select.
//  * scan_decode_kernel: the same contraction with key rows loaded straight into the B
//    operand; serves rows restricted to a candidate list (the hierarchical stage 2).
//  * scan_prefill_kernel (index_prefill.hip): many query rows (a prefill chunk), the one
//    dense contraction of the path.
//  * scan_generic_kernel: any head count/dim and fp32; one thread per candidate.
// Visibility: entry i is usable by a query at t only if m*(i+1)-1 <= t ("The sliding window
// is not an optimisation"); positions past a row's visible count are never scored.
#include <hip/hip_ext.h>
#include <stdlib.h>

#include "csa_common.hpp"
#include "index_common.hpp"
#include "ingest.hpp"
#include "launch.hpp"
#include "mxfp4.hpp"

namespace csa {

namespace {

// 16 MFMAs: acc[mt] = q[16 heads of mt] x key tile; then sum_h w_h * relu(acc)
__device__ __forceinline__ float tile_score(const bf16x8_t (&A)[4][4], const bf16x8_t (&B)[4],
                                            const float (&wv)[4][4]) {
  f32x4_t acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][ks], B[ks], acc[mt], 0, 0, 0);
  }
  float part = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) part = fmaf(wv[mt][i], relu_bits(acc[mt][i]), part);
  return sum_rows4(part);
}

template <bool NT>
__device__ __forceinline__ void load_key_B(const uint16_t* row, int g, bf16x8_t (&B)[4]) {
  const bf16x8_t* p = reinterpret_cast<const bf16x8_t*>(row + g * 8);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (NT) B[ks] = __builtin_nontemporal_load(p + 4 * ks);
    else B[ks] = p[4 * ks];
  }
}

// The wave that scores the entry a decode step completes pools its indexer key from the values
// a lane holds (channels 2*lane and 2*lane+1 of m rows, the new row in `slot`), stores it to
// the cache and puts it into the B operand of the key's column (patch_new_key; for an MXFP4
// cache into the code chunks and scale bytes read for it, patch_new_key_q4).
constexpr int kFuseM = 8;   // entries of up to 8 rows are pooled this way
// The pooled indexer key of entry e (row r): the channel-wise softmax over the block's m rows
// (the new token's row in slot `slot`, the tail's in the others), rounded to bf16; lane holds
// channels 2 lane, 2 lane + 1 of the packed result. The loads (load_new_key) and the
// arithmetic (pool_loaded_key) are separate steps, so that a caller can issue the loads
// before other memory traffic.
struct NewKeyIn {
  uint32_t xn, zn, xt[kFuseM], zt[kFuseM], bb[kFuseM];
};
__device__ __forceinline__ void load_new_key(const IngestArgs& ig, int64_t r, int slot, int lane,
                                             NewKeyIn& in) {
  const int m = ig.m;
  in.xn = reinterpret_cast<const uint32_t*>(ig.xi_new)[r * (kID / 2) + lane];
  in.zn = reinterpret_cast<const uint32_t*>(ig.zi_new)[r * (kID / 2) + lane];
#pragma unroll
  for (int j = 0; j < kFuseM; ++j) {
    in.xt[j] = in.zt[j] = in.bb[j] = 0u;
    if (j < m && j != slot) {
      in.xt[j] = reinterpret_cast<const uint32_t*>(ig.xi_tail)[(r * m + j) * (kID / 2) + lane];
      in.zt[j] = reinterpret_cast<const uint32_t*>(ig.zi_tail)[(r * m + j) * (kID / 2) + lane];
    }
    if (j < m) in.bb[j] = reinterpret_cast<const uint32_t*>(ig.bias_i)[j * (kID / 2) + lane];
  }
}
__device__ __forceinline__ uint32_t pool_loaded_key(const NewKeyIn& in, int m, int slot) {
  float res[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    auto half = [&](uint32_t w2) {
      return bf16_to_f32(uint16_t(h ? (w2 >> 16) : (w2 & 0xffffu)));
    };
    float av[kFuseM], mx = neg_inf();
#pragma unroll
    for (int j = 0; j < kFuseM; ++j) {
      av[j] = neg_inf();
      if (j < m) {
        av[j] = half(j == slot ? in.zn : in.zt[j]) + half(in.bb[j]);
        mx = fmaxf(mx, av[j]);
      }
    }
    float sum = 0.f, acc = 0.f;
#pragma unroll
    for (int j = 0; j < kFuseM; ++j)
      if (j < m) {
        const float ex = expf(av[j] - mx);
        sum += ex;
        acc = fmaf(ex, half(j == slot ? in.xn : in.xt[j]), acc);
      }
    res[h] = acc / sum;
  }
  return uint32_t(f32_to_bf16(res[0])) | (uint32_t(f32_to_bf16(res[1])) << 16);
}
__device__ __forceinline__ uint32_t pool_new_key(const IngestArgs& ig, int64_t r, int slot,
                                                 int lane) {
  NewKeyIn in;
  load_new_key(ig, r, slot, lane, in);
  return pool_loaded_key(in, ig.m, slot);
}

// bf16 cache: the pooled key is stored as it is
__device__ __forceinline__ uint32_t store_new_key(const IngestArgs& ig, int64_t r, int64_t e,
                                                  uint32_t pk, int lane) {
  reinterpret_cast<uint32_t*>(ig.k_idx)[(r * ig.e_cap + e) * (kID / 2) + lane] = pk;
  return pk;
}
__device__ __forceinline__ uint32_t fuse_new_key(const IngestArgs& ig, int64_t r, int64_t e,
                                                 int slot, int lane) {
  return store_new_key(ig, r, e, pool_new_key(ig, r, slot, lane), lane);
}

// MXFP4 cache: the pooled (bf16) key is quantised as csa_quantize_mxfp4 does it -- block b =
// channels 32 b .. 32 b + 31 = lanes 16 b .. 16 b + 15, whose maximum is a 16-lane DPP maximum
// of the magnitudes' bits -- and stored (lane l writes code byte l, lane 16 b the scale byte of
// block b). Returns code byte l in bits 0-7 and the scale byte of the lane's block in bits 8-15.
__device__ __forceinline__ uint32_t store_new_key_q4(const IngestArgs& ig, int64_t r, int64_t e,
                                                     uint32_t pk, int lane) {
  const float lo = bf16_to_f32(uint16_t(pk & 0xffffu)), hi = bf16_to_f32(uint16_t(pk >> 16));
  const uint32_t am = max16_key(__builtin_elementwise_max(__float_as_uint(fabsf(lo)),
                                                          __float_as_uint(fabsf(hi))));
  const int s = mx_shared_exp(__uint_as_float(am));
  const uint32_t code = e2m1_code(ldexpf(lo, -s)) | (e2m1_code(ldexpf(hi, -s)) << 4);
  const uint32_t sb = uint32_t(s + 127);
  const int64_t key = r * ig.e_cap + e;
  static_cast<uint8_t*>(ig.k_idx)[key * (kID / 2) + lane] = uint8_t(code);
  if ((lane & 15) == 0) static_cast<uint8_t*>(ig.k_scale)[key * (kID / 32) + (lane >> 4)] = uint8_t(sb);
  return code | (sb << 8);
}

// The B operand of the lanes that hold the new entry's key (mine: its column) from the packed
// key pk (channels 2 l, 2 l + 1 in lane l): the tile was loaded before the key was written.
// Lane (g, col) of k-step ks holds channels ks*32 + g*8 .. +8, from lanes ks*16 + g*4 + 0..3.
__device__ __forceinline__ void patch_new_key(uint32_t pk, int g, bool mine, bf16x8_t (&B)[4]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint32_t wds[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) wds[k] = uint32_t(__shfl(int(pk), ks * 16 + g * 4 + k));
    if (mine) B[ks] = *reinterpret_cast<const bf16x8_t*>(wds);
  }
}

// Candidate segment of one work item (row r, chunk c = positions [c0, c1)), from the scores
// the item left in LDS. tau = the J-th largest 16-position maximum with its low 12 bits
// cleared (J from the row's chunk count, well above the mean share K / chunks of the row's
// Top-K); every position whose key reaches tau is kept, in position order. Called by all
// threads of the block; ends with a barrier.
struct SegLds {
  float sc[kSegMaxChunk];
  uint32_t gm[kSegMaxChunk / 16];
  uint32_t red[8];
};
// Inclusive prefix sum over the 64 lanes with DPP: shifts by 1, 2, 4, 8 within each 16-lane
// row, then the row totals are carried by the row broadcasts (lane 15 into rows 1 and 3, lane
// 31 into rows 2 and 3). No LDS permutes.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x111, 0xf, 0xf, false));   // row_shr:1
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x112, 0xf, 0xf, false));   // row_shr:2
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x114, 0xf, 0xf, false));   // row_shr:4
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x118, 0xf, 0xf, false));   // row_shr:8
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x142, 0xa, 0xf, false));   // row_bcast:15
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x143, 0xc, 0xf, false));   // row_bcast:31
  return x;
}

// maximum over the 64 lanes: the 16-lane row maximum, then the two row swaps
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t k) {
  k = max16_key(k);
  const auto p = __builtin_amdgcn_permlane16_swap(k, k, false, false);
  k = __builtin_elementwise_max(uint32_t(p[0]), uint32_t(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(k, k, false, false);
  return __builtin_elementwise_max(uint32_t(q[0]), uint32_t(q[1]));
}

// J of the segment rule for an item of n visible positions in a row of n_pos (> 0): lambda =
// K / chunks is the mean count of the row's Top-K per chunk (positions are exchangeable);
// J = lambda + 4 sqrt(lambda) + 5 sits far in the Poisson tail; at most half the item's
// 16-position groups and at most 64, at least 1. 32-bit arithmetic (a row holds < 2^31 entries).
__device__ __forceinline__ int segment_quota(const SegArgs& sg, int64_t n_pos, int n) {
  const int ng = (n + 15) >> 4;
  const uint32_t ch = uint32_t(sg.chunk);
  uint32_t nch = (uint32_t(n_pos) + ch - 1u) / ch;
  nch = nch > 0u ? nch : 1u;
  const float lam = float(sg.K) / float(nch);
  int J = int(lam + 4.f * sqrtf(lam)) + 5;
  const int jmax = ng / 2 < 64 ? ng / 2 : 64;
  J = J > jmax ? jmax : J;
  return J < 1 ? 1 : J;
}

__device__ __forceinline__ void emit_segment(const SegArgs& sg, SegLds& L, int64_t r, int64_t c,
                                             int64_t c0, int64_t c1, int64_t n_pos,
                                             float* scores_row = nullptr, int J = 0) {
  __syncthreads();
  const int tid = int(threadIdx.x);
  const int lane = tid & 63, wave = tid >> 6;
  const int n = int(c1 - c0);
  const int ng = (n + 15) >> 4;
  const uint32_t kninf = order_key(neg_inf());
  // keys of 8 consecutive positions per thread (n <= 2048 = 256 threads x 8); the maximum
  // of a 16-position group from this thread and its neighbour
  const int i0 = tid * 8;
  uint32_t k[8];
  uint32_t km = 0u;
  if (i0 + 8 <= n) {
    const float4 a0 = *reinterpret_cast<const float4*>(&L.sc[i0]);
    const float4 a1 = *reinterpret_cast<const float4*>(&L.sc[i0 + 4]);
    if (scores_row) {
      float4* o = reinterpret_cast<float4*>(scores_row + c0 + i0);
      o[0] = a0;
      o[1] = a1;
    }
    k[0] = order_key(a0.x); k[1] = order_key(a0.y); k[2] = order_key(a0.z); k[3] = order_key(a0.w);
    k[4] = order_key(a1.x); k[5] = order_key(a1.y); k[6] = order_key(a1.z); k[7] = order_key(a1.w);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      k[i] = i0 + i < n ? order_key(L.sc[i0 + i]) : 0u;
      if (scores_row && i0 + i < n) scores_row[c0 + i0 + i] = L.sc[i0 + i];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) km = k[i] > km ? k[i] : km;
  const uint32_t kn = uint32_t(__builtin_amdgcn_update_dpp(0, int(km), 0xb1, 0xf, 0xf, false));
  km = kn > km ? kn : km;   // quad_perm [1,0,3,2]: the neighbour lane
  if ((tid & 1) == 0 && (i0 >> 4) < ng) L.gm[i0 >> 4] = km;
  __syncthreads();
  if (wave == 0) {
    // J: the caller's (computed ahead, off the item's critical path) or computed here
    if (J <= 0) J = segment_quota(sg, n_pos, n);
    const uint32_t v0 = lane < ng ? L.gm[lane] : 0u;
    const uint32_t v1 = lane + 64 < ng ? L.gm[lane + 64] : 0u;
    uint32_t x = 0u;
#pragma unroll
    for (int b = 31; b >= 12; --b) {
      const uint32_t y = x | (1u << b);
      const int cnt = __popcll(__ballot(v0 >= y)) + __popcll(__ballot(v1 >= y));
      if (cnt >= J) x = y;
    }
    const uint32_t mx = wave_max_u32(v0 > v1 ? v0 : v1);
    if (lane == 0) { L.red[0] = x; L.red[1] = mx; }
  }
  __syncthreads();
  const uint32_t tau = L.red[0];
  uint32_t flags = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i0 + i < n && k[i] >= tau && k[i] > kninf) flags |= 1u << i;
  const uint32_t cnt = __popc(flags);
  const uint32_t x = wave_incl_scan(cnt);
  if (lane == 63) L.red[2 + wave] = x;
  __syncthreads();
  uint32_t off = x - cnt, total = 0;
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) {
    const uint32_t t = L.red[2 + w2];
    if (w2 < wave) off += t;
    total += t;
  }
  const int64_t sidx = r * sg.nseg + c;
  uint2* dst = sg.seg + sidx * kChunkSegCap;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if ((flags >> i) & 1u) {
      if (off < uint32_t(kChunkSegCap)) dst[off] = make_uint2(k[i], uint32_t(c0 + i0 + i));
      ++off;
    }
  if (tid == 0) {
    sg.seg_n[sidx] = int32_t(total);
    sg.seg_info[sidx] = make_uint2(tau, L.red[1]);
  }
  __syncthreads();
}

}  // namespace

// Persistent grid: work item it = (row, chunk) = (it / cpr, it % cpr), chunk positions
// [c*chunk, (c+1)*chunk); blocks stride over the items, so the grid is sized to the machine
// rather than to the work (no partially filled last wave of blocks). Within an item, wave w
// scores 16-key tiles w, w+4, ... and keeps PF further tiles of keys in flight (registers)
// while the MFMAs of the current tile run.
// kSeg: the item's scores also go to LDS and the item ends with its candidate segment
// (emit_segment) instead of 16-position maxima in global memory.
template <bool kCand, int PF, bool NT, bool kSeg>
__global__ __launch_bounds__(256) void scan_decode_kernel(ScanArgs a, int chunk, int64_t cpr,
                                                          int64_t n_items) {
  __shared__ SegLds segl;   // used only when kSeg
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  bf16x8_t A[4][4];
  float wv[4][4];
  int64_t cur = -1;
  const bool fuse = !kCand && a.ingest.pos != nullptr;
  for (int64_t it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int64_t r = it / cpr, c = it % cpr;
    const int64_t n_vis = row_visible(a, r);
    const int64_t n_pos = kCand ? a.n_cand : n_vis;
    if (c == 0 && threadIdx.x == 0) {
      a.n_vis[r] = int32_t(n_vis);
      a.count[r] = int32_t(n_pos);
    }
    const int64_t c0 = c * chunk;
    if (c0 >= n_pos) continue;
    const int64_t c1 = c0 + chunk < n_pos ? c0 + chunk : n_pos;
    if (r != cur) {
      load_query_A(reinterpret_cast<const uint16_t*>(a.q) + r * kIH * kID, lane, A);
      load_gates(a.w + r * kIH, lane, wv);
      cur = r;
    }
    const int64_t sq = r / a.n_q;
    const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.keys) + sq * a.e_cap * kID;
    const int32_t* cand = kCand ? a.cand + r * a.n_cand : nullptr;
    float* out = a.scores + r * a.score_stride;
    uint32_t* gmax = a.gmax + r * a.gmax_stride;
    // key row of position p (positions past the chunk read a safe row and are not stored)
    auto key_row = [&](int64_t p, bool& ok) -> int64_t {
      if (p >= c1) { ok = false; return kCand ? 0 : c0; }
      if (kCand) {
        const int32_t id = cand[p];
        ok = id >= 0 && id < n_vis;
        return ok ? id : 0;
      }
      ok = true;
      return p;
    };
    // Decode ingest folded in: the entry that the step's token completes is pooled (now) by
    // the wave that scores it; lane shuffles place the key in the B operand of its column.
    int64_t e_new = -1;
    uint32_t pk_new = 0u;
    if (fuse) {
      const int64_t t = a.ingest.pos[r];
      const int64_t e = (t + 1) / a.ingest.m - 1;
      if (t >= 0 && (t + 1) % a.ingest.m == 0 && e >= c0 && e < c1 &&
          int((e - c0) >> 4) % 4 == wave) {
        e_new = e;
        pk_new = fuse_new_key(a.ingest, r, e, int(t % a.ingest.m), lane);
      }
    }
    const int64_t t0 = c0 + wave * 16;
    if (t0 < c1) {
      bf16x8_t buf[PF + 1][4];
      bool ok[PF + 1];
#pragma unroll
      for (int u = 0; u <= PF; ++u) {
        const int64_t tl = t0 + int64_t(u) * 64;
        load_key_B<NT>(kb + key_row(tl + col, ok[u]) * kID, g, buf[u]);
      }
      bool more = true;
      for (int64_t k = 0; more; k += PF + 1) {
#pragma unroll
        for (int u = 0; u <= PF; ++u) {
          const int64_t tl = t0 + (k + u) * 64;
          if (more && tl < c1) {
            if (e_new >= tl && e_new < tl + 16)
              patch_new_key(pk_new, g, col == int(e_new - tl), buf[u]);
            const float s = tile_score(A, buf[u], wv);
            const int64_t p = tl + col;
            const float sv = (p < c1 && ok[u]) ? s : neg_inf();
            if (g == 0 && p < c1) {
              out[p] = sv;
              if (kSeg) segl.sc[p - c0] = sv;
            }
            if (!kSeg) {
              const uint32_t gm = max16_key(order_key(sv));
              if (lane == 0) gmax[tl >> 4] = gm;
            }
            const int64_t nx = tl + int64_t(PF + 1) * 64;
            if (nx < c1) load_key_B<NT>(kb + key_row(nx + col, ok[u]) * kID, g, buf[u]);
          } else {
            more = false;
          }
        }
      }
    }
    if (kSeg) emit_segment(a.seg, segl, r, c, c0, c1, n_pos);
  }
}

// ---- decode scan with keys staged through LDS ------------------------------------------------
// The same contraction as scan_decode_kernel, for the whole visible range of each row (no
// candidate list), with the key rows moved by global_load_lds_dwordx4: each instruction
// reads 1 KiB of consecutive memory (4 key rows) straight into LDS, so every request covers
// whole cache lines, and no VGPRs hold keys in flight. A wave keeps kSD 16-key tiles in
// flight in a ring of LDS slots. Lane l of instruction i of a tile loads the 16-byte chunk
// l >> 2 of key 4i + (l & 3) into slot byte 16 l of the instruction's 1 KiB block; blocks are
// 1,088 bytes apart, which makes the B-operand reads (lane (g, col) of k-step ks reads chunk
// 4 ks + g of key col) hit 16 distinct 4-bank groups per quarter-wave. The channel order
// is that of load_key_B, so the query operand is unchanged. A tile is read only after the
// wave's memory counter shows its loads done (loads complete in issue order; every wait
// counts only the tile loads issued after it, so any other memory operation in between only
// makes it wait longer). Scores stay in LDS and leave in one coalesced pass per item, then the
// item's candidate segment (kSeg) or its 16-position maxima.
constexpr int kTileLds = 4 * kBlk;         // LDS bytes per 16-key tile

typedef __attribute__((address_space(3))) void lds_void;

template <bool NT>
__device__ __forceinline__ void issue_tile(const uint16_t* kb, int64_t tb, int64_t lim,
                                           unsigned char* slot, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t key = tb + 4 * i + (lane & 3);
    key = key < lim ? key : lim - 1;   // rows past the item read its last row (discarded)
    __builtin_amdgcn_global_load_lds(kb + key * kID + (lane >> 2) * 8,
                                     (lds_void*)(slot + i * kBlk), 16, 0, NT ? 2 : 0);
  }
}

// B operand of the tile in `slot` once at most 4 n tile loads of this wave are outstanding
// (n = tiles issued after this one, 0 <= n < kSD, wave-uniform). The wait and the four LDS
// reads are one asm block: the compiler's own wait insertion would otherwise wait for every
// outstanding load before any read of LDS written by global_load_lds.
#define CSA_TILE_READ(VM)                                                                   \
  asm volatile("s_waitcnt vmcnt(" #VM ")\n\t"                                              \
               "ds_read_b128 %0, %4\n\t"                                                   \
               "ds_read_b128 %1, %4 offset:256\n\t"                                        \
               "ds_read_b128 %2, %4 offset:512\n\t"                                        \
               "ds_read_b128 %3, %4 offset:768\n\t"                                        \
               "s_waitcnt lgkmcnt(0)"                                                      \
               : "=&v"(B[0]), "=&v"(B[1]), "=&v"(B[2]), "=&v"(B[3])                            \
               : "v"(addr)                                                                 \
               : "memory")
__device__ __forceinline__ void read_tile_B(const unsigned char* slot, int g, int col, int n,
                                            bf16x8_t (&B)[4]) {
  const unsigned char* base = slot + (col >> 2) * kBlk + (col & 3) * 16 + g * 64;
  const uint32_t addr = uint32_t(size_t((const __attribute__((address_space(3))) unsigned char*)base));
  switch (__builtin_amdgcn_readfirstlane(n)) {
    case 0: CSA_TILE_READ(0); break;
    case 1: CSA_TILE_READ(4); break;
    case 2: CSA_TILE_READ(8); break;
    default: CSA_TILE_READ(12); break;
  }
}
#undef CSA_TILE_READ

// ---- MXFP4 keys: 64-key tiles ---------------------------------------------------------------
// Keys as csa_quantize_mxfp4 stores them: 64 code bytes per key (element 2i in the low nibble
// of byte i) and 4 scale bytes (one per 32 channels). A wave's tile is 64 keys: 4 KiB of codes
// by four global_load_lds_dwordx4 (one per 16-key group) and the 256 scale bytes by one
// global_load_lds_dword -- the LDS footprint of a bf16 tile, four times the keys. In the MFMA
// lane (g, col) of k-step ks takes channels 32 g + 8 ks .. + 8, so a lane's four k-steps are one
// 16-byte chunk of key col's codes (chunk g) under one scale (block g); the query operand takes
// the same channel order (load_query_A_q4). Chunk g of key col of a group sits in 16-byte slot
// 4 col + ((col >> 2) + g) % 4: the 16 lanes of a quarter-wave (one g) read 16 distinct slots
// mod 16. Dequantisation is exact (an E2M1 value times a power of two is a bf16 value) by
// v_cvt_scalef32_pk_bf16_fp4, whose result holds the low nibble's value in its low half.
constexpr int kQ4Keys = 64;
constexpr int kQ4Codes = kQ4Keys * kID / 2;   // 4,096 code bytes, then 256 scale bytes
static_assert(kQ4Codes + kQ4Keys * kID / 32 <= kTileLds, "an MXFP4 tile fits a ring slot");

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

// A operand of one query in the MXFP4 channel order: heads 16*mt + (lane&15), channels
// 32 g + 8 ks .. + 8 (g = lane >> 4)
__device__ __forceinline__ void load_query_A_q4(const uint16_t* q, int lane, bf16x8_t (&A)[4][4]) {
  const int g = lane >> 4, col = lane & 15;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const uint16_t* p = q + (16 * mt + col) * kID + g * 32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) A[mt][ks] = *reinterpret_cast<const bf16x8_t*>(p + ks * 8);
  }
}

// codes of key tb + 16 i + (lane >> 2), chunk ((lane & 3) - (lane >> 4)) % 4, into slot byte
// 1024 i + 16 lane; scales of key tb + lane into byte 4096 + 4 lane. Keys at or past lim read
// the item's last key (discarded).
template <bool NT>
__device__ __forceinline__ void issue_tile_q4(const uint8_t* cb, const uint8_t* sb, int64_t tb,
                                              int64_t lim, unsigned char* slot, int lane) {
  const int kc = lane >> 2;
  const int ch = ((lane & 3) - (kc >> 2)) & 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t key = tb + 16 * i + kc;
    key = key < lim ? key : lim - 1;
    __builtin_amdgcn_global_load_lds(cb + key * (kID / 2) + ch * 16,
                                     (lds_void*)(slot + i * 1024), 16, 0, NT ? 2 : 0);
  }
  int64_t key = tb + lane;
  key = key < lim ? key : lim - 1;
  __builtin_amdgcn_global_load_lds(sb + key * (kID / 32), (lds_void*)(slot + kQ4Codes), 4, 0,
                                   NT ? 2 : 0);
}

// The codes chunk and scale byte of this lane for the four 16-key groups of the tile in `slot`,
// once at most 5 n tile loads of this wave are outstanding (n tiles issued after this one).
#define CSA_Q4_READ(VM)                                                                      \
  asm volatile("s_waitcnt vmcnt(" #VM ")\n\t"                                               \
               "ds_read_b128 %0, %8\n\t"                                                    \
               "ds_read_b128 %1, %8 offset:1024\n\t"                                        \
               "ds_read_b128 %2, %8 offset:2048\n\t"                                        \
               "ds_read_b128 %3, %8 offset:3072\n\t"                                        \
               "ds_read_u8 %4, %9\n\t"                                                      \
               "ds_read_u8 %5, %9 offset:64\n\t"                                            \
               "ds_read_u8 %6, %9 offset:128\n\t"                                           \
               "ds_read_u8 %7, %9 offset:192\n\t"                                           \
               "s_waitcnt lgkmcnt(0)"                                                       \
               : "=&v"(cw[0]), "=&v"(cw[1]), "=&v"(cw[2]), "=&v"(cw[3]), "=&v"(sc[0]),     \
                 "=&v"(sc[1]), "=&v"(sc[2]), "=&v"(sc[3])                                   \
               : "v"(caddr), "v"(saddr)                                                     \
               : "memory")
__device__ __forceinline__ void read_tile_q4(const unsigned char* slot, int g, int col, int n,
                                             u32x4_t (&cw)[4], uint32_t (&sc)[4]) {
  typedef const __attribute__((address_space(3))) unsigned char* lds_cptr;
  const uint32_t caddr = uint32_t(size_t((lds_cptr)(slot + 16 * (4 * col + (((col >> 2) + g) & 3)))));
  const uint32_t saddr = uint32_t(size_t((lds_cptr)(slot + kQ4Codes + 4 * col + g)));
  switch (__builtin_amdgcn_readfirstlane(n)) {
    case 0: CSA_Q4_READ(0); break;
    case 1: CSA_Q4_READ(5); break;
    case 2: CSA_Q4_READ(10); break;
    default: CSA_Q4_READ(15); break;
  }
}
#undef CSA_Q4_READ

// B operand (bf16) of one 16-key group from this lane's code chunk and scale byte (a scale
// byte of 0 is 2^-127, a subnormal float)
__device__ __forceinline__ void dequant_B(const u32x4_t cw, uint32_t sbyte, bf16x8_t (&B)[4]) {
  const float s = __uint_as_float(sbyte ? sbyte << 23 : 0x00400000u);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint32_t w = cw[ks];
    uint32_t o[4];
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3));
    B[ks] = __builtin_bit_cast(bf16x8_t, o);
  }
}

// FP4 query-key path: the query as MXFP4 (the keys' rule, mxfp4.hpp), one 32-channel block per
// thread of the workgroup (64 heads x 4 blocks = 256): thread t quantises head t / 4, channels
// 32 (t % 4) .. + 31 into qc[t] (16 code bytes, channel 32 (t % 4) + k in nibble k of dword
// k / 8, the key chunks' order) and qs[t] (its scale byte). The caller publishes them with a
// barrier; lane (g, col) of the MFMA then takes block 4 (16 mt + col) + g as A[mt].
// the block's 32 bf16 values, two per word (low half first)
__device__ __forceinline__ void load_query_block(const uint16_t* q, int t, uint32_t (&w)[16]) {
  const uint4* p = reinterpret_cast<const uint4*>(q + (t >> 2) * kID + 32 * (t & 3));
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 v = p[c];
    w[4 * c] = v.x; w[4 * c + 1] = v.y; w[4 * c + 2] = v.z; w[4 * c + 3] = v.w;
  }
}
__device__ __forceinline__ void quantize_query_block(const uint32_t (&w)[16], int t, uint4* qc,
                                                     uint8_t* qs) {
  // the largest magnitude: an integer maximum of the magnitude bits (monotone for bf16)
  uint32_t mb = 0u;
#pragma unroll
  for (int k = 0; k < 16; ++k)
    mb = __builtin_elementwise_max(mb, __builtin_elementwise_max(w[k] & 0x7fffu,
                                                                 (w[k] >> 16) & 0x7fffu));
  const int s = mx_shared_exp(__uint_as_float(mb << 16));
  // 2^-s: a normal float for s >= -126, 2^127 for s = -127
  const float inv = __uint_as_float(uint32_t(s > -127 ? 127 - s : 254) << 23);
  uint32_t code[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    code[d] = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      code[d] |= e2m1_code(bf16_lo(w[4 * d + k]) * inv) << (8 * k);
      code[d] |= e2m1_code(bf16_hi(w[4 * d + k]) * inv) << (8 * k + 4);
    }
  }
  qc[t] = make_uint4(code[0], code[1], code[2], code[3]);
  qs[t] = uint8_t(s + 127);
}

// The 4 MFMAs of one 16-key group on the FP4 query-key path: acc[mt] = the FP4 query heads of
// mt x the group's FP4 keys (code chunk and scale byte of this lane), K = 128 in one
// instruction; the products of two FP4 values under power-of-two scales are exact.
__device__ __forceinline__ void tile_mfma_fp4(const u32x4_t (&A)[4], const uint32_t (&sa)[4],
                                              const u32x4_t cw, uint32_t sb, f32x4_t (&acc)[4]) {
  typedef int v8i_t __attribute__((ext_vector_type(8)));
  const v8i_t b = {int(cw[0]), int(cw[1]), int(cw[2]), int(cw[3]), 0, 0, 0, 0};
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const v8i_t am = {int(A[mt][0]), int(A[mt][1]), int(A[mt][2]), int(A[mt][3]), 0, 0, 0, 0};
    acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        am, b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, int(sa[mt]), 0, int(sb));
  }
}

// The code chunk and scale byte of the lanes that hold the new entry (its group and column,
// from its offset off in the tile): the tile was loaded before the entry was written. v holds
// code byte l of the entry in lane l and the scale byte of the lane's block; lane (g, col)
// takes bytes 16 g .. 16 g + 15 (lanes 16 g + 4 ks + k) and the scale of block g, its own.
__device__ __forceinline__ void patch_new_key_q4(uint32_t v, int off, int g, int col,
                                                 u32x4_t (&cw)[4], uint32_t (&sc)[4]) {
  u32x4_t w;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint32_t x = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) x |= (uint32_t(__shfl(int(v), g * 16 + ks * 4 + k)) & 0xffu) << (8 * k);
    w[ks] = x;
  }
  const bool mine = col == (off & 15);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (mine && j == (off >> 4)) {
      cw[j] = w;
      sc[j] = v >> 8;
    }
}

// kQ4: MXFP4 keys (a.key_scales), 64-key tiles; else bf16 keys, 16-key tiles. kQK (with kQ4):
// the query quantised to MXFP4 as well, the products taken by the FP4 MFMA.
template <bool NT, bool kSeg, int kSD, bool kQ4, bool kQK = false>
__global__ __launch_bounds__(256, 2) void scan_stream_kernel(ScanArgs a, int chunk, int64_t cpr,
                                                          int64_t n_items, int rot) {
  static_assert(kQ4 || !kQK, "the FP4 query-key path reads MXFP4 keys");
  constexpr int kTK = kQ4 ? kQ4Keys : 16;   // keys per wave tile
  __shared__ __attribute__((aligned(16))) unsigned char ring[4][kSD][kTileLds];
  __shared__ SegLds segl;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  bf16x8_t A[4][4];
  u32x4_t A4[4];
  uint32_t sa4[4];
  float wv[4][4];
  int64_t cur = -1;
  const bool fuse = a.ingest.pos != nullptr;
  for (int64_t it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int64_t r = it / cpr, c = it % cpr;
    const int64_t sq = r / a.n_q;
    const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.keys) + sq * a.e_cap * kID;
    const uint8_t* cb = reinterpret_cast<const uint8_t*>(a.keys) + sq * a.e_cap * (kID / 2);
    const uint8_t* sb = a.key_scales + sq * a.e_cap * (kID / 32);
    const int64_t c0 = c * chunk;
    const int64_t lim = c0 + chunk < a.e_cap ? c0 + chunk : a.e_cap;
    // wave w takes the tiles w, w + 4, ... of the item in the order that starts at tile `r0`
    // (a per-block rotation, so that blocks do not walk memory in step)
    const int64_t t0 = c0 + wave * kTK;
    const int nt_item = int((lim - t0 + 4 * kTK - 1) / (4 * kTK));   // tiles of this wave
    const int r0 = nt_item > 0 ? int((int64_t(blockIdx.x) * rot) % nt_item) : 0;
    auto tile_base = [&](int t) -> int64_t {
      int u = t + r0;
      u = u >= nt_item ? u - nt_item : u;
      return t0 + int64_t(u) * (4 * kTK);
    };
    auto issue = [&](int t, unsigned char* slot) {
      if (kQ4) issue_tile_q4<NT>(cb, sb, tile_base(t), lim, slot, lane);
      else issue_tile<NT>(kb, tile_base(t), lim, slot, lane);
    };
    // The row's visible count, query and gates, and the inputs of the entry this step's token
    // completes (pooled by the wave that scores it), are loaded before the first tiles: a wave's
    // loads return in issue order, so loads issued after the tiles would wait for them. The FP4
    // query is quantised after the first tiles have gone out, while they are in flight.
    // The row's position is a scalar load (r is uniform; positions are inputs no kernel of the
    // step writes): its wait counts scalar loads only, so the query loads and the first tiles
    // go out without waiting for it (as a vector load, its value taken into scalar registers
    // would first wait for every vector load before it).
    const int64_t t_row = *(const __attribute__((address_space(4))) int64_t*)(a.q_pos + r);
    uint32_t qw[16];
    const bool new_row = r != cur;   // uniform over the block
    if (new_row) {
      const uint16_t* qr = reinterpret_cast<const uint16_t*>(a.q) + r * kIH * kID;
      if (kQK) load_query_block(qr, int(threadIdx.x), qw);
      else if (kQ4) load_query_A_q4(qr, lane, A);
      else load_query_A(qr, lane, A);
      load_gates(a.w + r * kIH, lane, wv);
      cur = r;
    }
    const int64_t n_pos = row_visible_at(a, r, t_row);
    const int64_t c1 = lim < n_pos ? lim : n_pos;
    // the segment rule's J for this item, formed now while the first tiles are in flight (the
    // empty asm keeps it ahead of the tile loop rather than sunk into the emission)
    int seg_J = 0;
    if (kSeg) {
      seg_J = __builtin_amdgcn_readfirstlane(segment_quota(a.seg, n_pos, int(c1 > c0 ? c1 - c0 : 0)));
      asm volatile("" : "+s"(seg_J));
    }
    int64_t e_new = -1;
    int new_slot = 0;
    NewKeyIn nk;
    if (fuse && c0 < c1) {
      // the step's position: the value loaded with the visible count when the two arrays are
      // one (the decode step's), so that no load issued after the query's is waited for here
      const int64_t t = a.ingest.pos == a.q_pos ? t_row : a.ingest.pos[r];
      const int64_t e = (t + 1) / a.ingest.m - 1;
      if (t >= 0 && (t + 1) % a.ingest.m == 0 && e >= c0 && e < c1 &&
          int((e - c0) / kTK) % 4 == wave) {
        e_new = e;
        new_slot = int(t % a.ingest.m);
        load_new_key(a.ingest, r, new_slot, lane, nk);
      }
    }
    // Every one of the first kSD tiles goes out, a wave with fewer tiles reading the item's last
    // key into slots it never reads (its waits only grow stricter), so that the compiler can
    // count the loads issued after the query's and wait for those alone: were some of these
    // issues conditional, its count at the join could not tell the query from the tiles, and
    // the tile loop's first MFMAs would drain every load in flight, the prefetched tiles too.
#pragma unroll
    for (int j = 0; j < kSD; ++j) issue(j, ring[wave][j]);
    if constexpr (!kQK) {
      // the query operand and the gates, loaded before these tiles, waited for here alone
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) asm volatile("" ::"v"(A[i][j]), "v"(wv[i][j]));
    }
    if constexpr (kQK) {
      if (new_row) {
        __shared__ uint4 qc[kIH * 4];
        __shared__ uint8_t qs[kIH * 4];
        quantize_query_block(qw, int(threadIdx.x), qc, qs);
        __syncthreads();
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const uint4 v = qc[4 * (16 * mt + col) + g];
          A4[mt] = u32x4_t{v.x, v.y, v.z, v.w};
          sa4[mt] = qs[4 * (16 * mt + col) + g];
        }
        __syncthreads();   // every lane has its operands before a later row overwrites them
      }
    }
    if (c == 0 && threadIdx.x == 0) {
      a.n_vis[r] = int32_t(n_pos);
      a.count[r] = int32_t(n_pos);
    }
    if (c0 < c1) {
      uint32_t pk_new = 0u;
      if (e_new >= 0) {
        const uint32_t pk = pool_loaded_key(nk, a.ingest.m, new_slot);
        pk_new = kQ4 ? store_new_key_q4(a.ingest, r, e_new, pk, lane)
                     : store_new_key(a.ingest, r, e_new, pk, lane);
      }
      // The first kSD tiles go out before the visible count is known; after that a tile is
      // issued only when it starts before the visible end c1, so a ragged row loads no tiles
      // past its end. Tiles land in issue order: tile t waits for all but the tiles issued
      // after it, those of t + 1 .. t + kSD - 1 that were issued (tile t + kSD goes out after
      // tile t is read). A tile issued past c1 is waited for (its slot is reused) but not
      // scored.
      const bool full = c1 >= lim;   // the whole item is visible: every tile goes out
      auto was_issued = [&](int j) { return full || j < kSD || tile_base(j) < c1; };
      for (int t = 0; t < nt_item; ++t) {
        const int64_t tb = tile_base(t);
        unsigned char* slot = ring[wave][t % kSD];
        int later = 0;
#pragma unroll
        for (int k = 1; k < kSD; ++k)
          if (t + k < nt_item && was_issued(t + k)) ++later;
        // a tile never issued (past c1; the order is rotated, so one issued later may follow
        // it) is neither read nor scored, and the issue below still runs
        if (!was_issued(t)) {   // uniform over the wave
        } else if constexpr (kQ4) {
          u32x4_t cw[4];
          uint32_t sc4[4];
          read_tile_q4(slot, g, col, later, cw, sc4);
          if (tb < c1) {
            if (e_new >= tb && e_new < tb + kQ4Keys)
              patch_new_key_q4(pk_new, int(e_new - tb), g, col, cw, sc4);
            // group j's MFMAs go out (into the other accumulator set) before the epilogue of
            // group j - 1, so the matrix pipe works while the VALU reduces; the head sums of
            // the four groups finish together (sum_groups4). Groups past the visible range
            // are scored too (their keys are the item's last one) and not stored.
            f32x4_t acc[2][4];
            float scb[4];
            if constexpr (kQK) {
              // FP4 x FP4: group j + 1's 4 MFMAs go out before the epilogue of group j, each
              // followed by a quarter of that epilogue
              tile_mfma_fp4(A4, sa4, cw[0], sc4[0], acc[0]);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                if (j + 1 < 4) tile_mfma_fp4(A4, sa4, cw[j + 1], sc4[j + 1], acc[(j + 1) & 1]);
                scb[j] = lane_part(acc[j & 1], wv);
                if (j + 1 < 4) {
#pragma unroll
                  for (int q = 0; q < 4; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                  }
                }
              }
            } else {
              bf16x8_t B[4];
              dequant_B(cw[0], sc4[0], B);
              tile_mfma(A, B, acc[0]);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                if (j + 1 < 4) {
                  dequant_B(cw[j + 1], sc4[j + 1], B);
                  tile_mfma(A, B, acc[(j + 1) & 1]);
                }
                scb[j] = lane_part(acc[j & 1], wv);
                if (j + 1 < 4) {
                  // issue order: the next group's 16 conversions, then each of its 16 MFMAs
                  // followed by two VALU instructions of this group's epilogue
                  __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
#pragma unroll
                  for (int q = 0; q < 16; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
                  }
                }
              }
            }
            const float sv = sum_groups4(scb[0], scb[1], scb[2], scb[3]);
            const int64_t p = tb + 16 * ((g & 1) * 2 + (g >> 1)) + col;   // row g: group grp
            if (p < c1) segl.sc[p - c0] = a.score_bf16 ? round_to_bf16(sv) : sv;
          }
        } else {
          bf16x8_t B[4];
          read_tile_B(slot, g, col, later, B);
          if (tb < c1) {
            if (e_new >= tb && e_new < tb + 16)
              patch_new_key(pk_new, g, col == int(e_new - tb), B);
            const float sc = tile_score(A, B, wv);
            const int64_t p = tb + col;
            if (g == 0 && p < c1) segl.sc[p - c0] = a.score_bf16 ? round_to_bf16(sc) : sc;
          }
        }
        if (t + kSD < nt_item && was_issued(t + kSD)) issue(t + kSD, slot);
      }
    }
    // tiles loaded past the visible range (or a row with none) must land before reuse
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (c0 >= c1) continue;   // uniform over the block
    if (kSeg) {
      emit_segment(a.seg, segl, r, c, c0, c1, n_pos, a.scores + r * a.score_stride, seg_J);
    } else {
      __syncthreads();
      float* out = a.scores + r * a.score_stride;
      const int n = int(c1 - c0);
      for (int i = threadIdx.x; i < n; i += 256) out[c0 + i] = segl.sc[i];
      uint32_t* gmax = a.gmax + r * a.gmax_stride;
      for (int gi = threadIdx.x; gi * 16 < n; gi += 256) {
        uint32_t mx = 0u;
        for (int i = gi * 16; i < gi * 16 + 16 && i < n; ++i) {
          const uint32_t k = order_key(segl.sc[i]);
          mx = k > mx ? k : mx;
        }
        gmax[(c0 >> 4) + gi] = mx;
      }
      __syncthreads();
    }
  }
}

// ---- generic: one thread per candidate position; any H <= 64, d <= 256, fp32 or bf16 ------
template <typename T>
__global__ __launch_bounds__(256) void scan_generic_kernel(ScanArgs a) {
  extern __shared__ float qs[];   // [H*d] query, then [H] gates
  const int64_t r = blockIdx.y;
  const int64_t n_vis = row_visible(a, r);
  const int64_t n_pos = a.cand ? a.n_cand : n_vis;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.n_vis[r] = int32_t(n_vis);
    a.count[r] = int32_t(n_pos);
  }
  const int64_t p = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (int64_t(blockIdx.x) * blockDim.x >= n_pos) return;   // uniform per block
  const int H = a.H, d = a.d;
  const T* q = reinterpret_cast<const T*>(a.q) + r * H * d;
  for (int i = threadIdx.x; i < H * d; i += blockDim.x) qs[i] = Elt<T>::load1(q + i);
  for (int i = threadIdx.x; i < H; i += blockDim.x) qs[H * d + i] = a.w[r * H + i];
  __syncthreads();
  const bool live = p < n_pos;
  int64_t id = p;
  bool ok = live;
  if (live && a.cand) {
    id = a.cand[r * a.n_cand + p];
    ok = id >= 0 && id < n_vis;
  }
  float s = neg_inf();
  if (ok) {
    const int64_t sq = r / a.n_q;
    const T* key = reinterpret_cast<const T*>(a.keys) + (sq * a.e_cap + id) * d;
    float dot[64];
#pragma unroll
    for (int h = 0; h < 64; ++h) dot[h] = 0.f;
    for (int c0 = 0; c0 < d; c0 += 8) {
      float kv8[8];
      Elt<T>::load8(key + c0, kv8);
#pragma unroll
      for (int h = 0; h < 64; ++h) {
        if (h < H) {
          const float* qh = qs + h * d + c0;
#pragma unroll
          for (int c = 0; c < 8; ++c) dot[h] = fmaf(qh[c], kv8[c], dot[h]);
        }
      }
    }
    s = 0.f;
#pragma unroll
    for (int h = 0; h < 64; ++h)
      if (h < H) s = fmaf(qs[H * d + h], fmaxf(dot[h], 0.f), s);
  }
  if (live) a.scores[r * a.score_stride + p] = s;
  // 16 consecutive positions sit in 16 consecutive lanes (block bases are multiples of 256)
  const uint32_t gm = max16_key(order_key(s));
  if ((threadIdx.x & 15) == 0 && live) a.gmax[r * a.gmax_stride + (p >> 4)] = gm;
}

static bool fast_shape(const ScanArgs& a) { return a.dt == kBF16 && a.H == kIH && a.d == kID; }

// Decode-scan launch shape: positions per work item, key tiles in flight per wave beyond the
// current one, and blocks resident per CU (the persistent grid is n_cu * blocks_per_cu).
struct ScanTune {
  int chunk = 2048, pf = 1, blocks_per_cu = 2, nt = 1, sd = 2, sd4 = 2, rot = 0;
  int prefill_q = 12, prefill_keys = 4096;
};
static int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return v ? atoi(v) : dflt;
}
static const ScanTune& scan_tune() {
  static const ScanTune t = [] {
    ScanTune x;
    x.chunk = env_int("CSA_TUNE_SCAN_CHUNK", x.chunk);
    x.pf = env_int("CSA_TUNE_SCAN_PF", x.pf);
    x.blocks_per_cu = env_int("CSA_TUNE_SCAN_BPC", x.blocks_per_cu);
    x.nt = env_int("CSA_TUNE_SCAN_NT", x.nt);
    x.sd = env_int("CSA_TUNE_SCAN_SD", x.sd);
    x.sd4 = env_int("CSA_TUNE_SCAN_SD4", x.sd4);
    x.rot = env_int("CSA_TUNE_SCAN_ROT", x.rot);
    x.prefill_q = env_int("CSA_TUNE_PREFILL_Q", x.prefill_q);
    x.prefill_keys = (env_int("CSA_TUNE_PREFILL_KEYS", x.prefill_keys) + 127) / 128 * 128;
    if (x.prefill_keys < 128) x.prefill_keys = 128;
    return x;
  }();
  return t;
}
static int n_cu() {
  static const int n = [] {
    int dev = 0, cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cu = 256;
    return cu > 0 ? cu : 256;
  }();
  return n;
}

static int64_t scan_grid() {
  const int bpc = scan_tune().blocks_per_cu > 0 ? scan_tune().blocks_per_cu : 2;
  return int64_t(n_cu()) * bpc;
}

// chunk: the tuned size (at most kSegMaxChunk with segments), shrunk (to >= 256 positions)
// until there is at least one work item per resident block
int decode_scan_chunk(int64_t rows, int64_t max_pos, bool segments) {
  const ScanTune& t = scan_tune();
  int chunk = t.chunk > 0 ? (t.chunk + 63) / 64 * 64 : 2048;
  if (segments && chunk > kSegMaxChunk) chunk = kSegMaxChunk;
  const int64_t grid = scan_grid();
  while (chunk > 256 && rows * ((max_pos + chunk - 1) / chunk) < grid) chunk /= 2;
  return (chunk + 63) / 64 * 64;
}

static size_t r256(size_t x) { return (x + 255) / 256 * 256; }

size_t seg_bytes(int64_t rows, int64_t max_pos) {
  const int chunk = decode_scan_chunk(rows, max_pos, true);
  const int64_t nseg = max_pos > 0 ? (max_pos + chunk - 1) / chunk : 1;
  const size_t ns = size_t(rows) * size_t(nseg);
  return r256(ns * kChunkSegCap * 8) + r256(ns * 4) + r256(ns * 8);
}

SegArgs seg_carve(void* base, int64_t rows, int64_t max_pos, int K) {
  SegArgs g;
  g.chunk = decode_scan_chunk(rows, max_pos, true);
  g.nseg = max_pos > 0 ? (max_pos + g.chunk - 1) / g.chunk : 1;
  g.K = K;
  const size_t ns = size_t(rows) * size_t(g.nseg);
  char* p = static_cast<char*>(base);
  g.seg = reinterpret_cast<uint2*>(p);
  g.seg_n = reinterpret_cast<int32_t*>(p + r256(ns * kChunkSegCap * 8));
  g.seg_info = reinterpret_cast<uint2*>(p + r256(ns * kChunkSegCap * 8) + r256(ns * 4));
  return g;
}

template <bool kCand, int PF, bool NT, bool kSeg>
static void launch_decode(const ScanArgs& a, int64_t rows, int64_t max_pos, hipStream_t s,
                          hipEvent_t e0, hipEvent_t e1) {
  int64_t grid = scan_grid();
  const int chunk = kSeg ? a.seg.chunk : decode_scan_chunk(rows, max_pos, false);
  const int64_t cpr = max_pos > 0 ? (max_pos + chunk - 1) / chunk : 1;
  const int64_t items = rows * cpr;
  if (grid > items) grid = items;
  launch_k(scan_decode_kernel<kCand, PF, NT, kSeg>, dim3(static_cast<unsigned>(grid)), dim3(256),
           0, s, e0, e1, a, chunk, cpr, items);
}

template <bool kCand, bool kSeg>
static void launch_decode_pf(const ScanArgs& a, int64_t rows, int64_t max_pos, hipStream_t s,
                             hipEvent_t e0, hipEvent_t e1) {
  const bool nt = scan_tune().nt != 0;
  switch (scan_tune().pf) {
    case 1: nt ? launch_decode<kCand, 1, true, kSeg>(a, rows, max_pos, s, e0, e1)
               : launch_decode<kCand, 1, false, kSeg>(a, rows, max_pos, s, e0, e1); break;
    case 3: nt ? launch_decode<kCand, 3, true, kSeg>(a, rows, max_pos, s, e0, e1)
               : launch_decode<kCand, 3, false, kSeg>(a, rows, max_pos, s, e0, e1); break;
    default: nt ? launch_decode<kCand, 2, true, kSeg>(a, rows, max_pos, s, e0, e1)
                : launch_decode<kCand, 2, false, kSeg>(a, rows, max_pos, s, e0, e1); break;
  }
}

bool scan_fuses_ingest(int dt, int H, int d, int m) {
  return dt == kBF16 && H == kIH && d == kID && m <= kFuseM;
}

bool scan_reads_mxfp4(int dt, int H, int d, int64_t n_q, bool cand) {
  return dt == kBF16 && H == kIH && d == kID && n_q < 16 && !cand;
}

template <bool kQ4, bool kQK = false>
static void launch_stream(const ScanArgs& a, int chunk, int64_t cpr, int64_t items, hipStream_t s,
                          hipEvent_t e0, hipEvent_t e1) {
  int64_t grid = scan_grid();
  if (grid > items) grid = items;
  const dim3 gd(static_cast<unsigned>(grid)), bd(256);
  const int rot = scan_tune().rot;
  const int sd = kQ4 ? scan_tune().sd4 : scan_tune().sd;
  const bool segs = a.seg.seg != nullptr;
#define CSA_STREAM(SEG, SD)                                                                  \
  launch_k(scan_stream_kernel<true, SEG, SD, kQ4, kQK>, gd, bd, 0, s, e0, e1, a, chunk, cpr, items, \
           rot)
  if (segs) {
    if (sd == 2) CSA_STREAM(true, 2);
    else if (sd == 3) CSA_STREAM(true, 3);
    else CSA_STREAM(true, 4);
  } else {
    if (sd == 2) CSA_STREAM(false, 2);
    else if (sd == 3) CSA_STREAM(false, 3);
    else CSA_STREAM(false, 4);
  }
#undef CSA_STREAM
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int64_t rows = a.n_seq * a.n_q;
  if (rows == 0) return hipSuccess;
  const int64_t max_pos = a.cand ? a.n_cand : a.e_cap;
  const bool q4 = a.key_scales != nullptr;
  if ((q4 || a.score_bf16) && !scan_reads_mxfp4(a.dt, a.H, a.d, a.n_q, a.cand != nullptr))
    return hipErrorInvalidValue;
  if (a.q_fp4 && !q4) return hipErrorInvalidValue;
  if (!q4 && fast_shape(a) && a.cand == nullptr && a.n_q >= 16) {
    const int keys_per_block = scan_tune().prefill_keys;
    const int pq = scan_tune().prefill_q == 8 ? 8 : 12;
    const int64_t groups = a.n_seq * ((a.n_q + pq - 1) / pq);
    const dim3 grid(static_cast<unsigned>((a.e_cap + keys_per_block - 1) / keys_per_block),
                    static_cast<unsigned>(groups));
    return launch_scan_prefill(a, pq, keys_per_block, grid, s, e0, e1);
  }
  if (fast_shape(a)) {
    if (a.cand) {
      launch_decode_pf<true, false>(a, rows, max_pos, s, e0, e1);
    } else {
      const int chunk = a.seg.seg ? a.seg.chunk : decode_scan_chunk(rows, max_pos, true);
      if (chunk > kSegMaxChunk) return hipErrorInvalidValue;
      const int64_t cpr = (max_pos + chunk - 1) / chunk;
      const int64_t items = rows * cpr;
      if (q4 && a.q_fp4) launch_stream<true, true>(a, chunk, cpr, items, s, e0, e1);
      else if (q4) launch_stream<true>(a, chunk, cpr, items, s, e0, e1);
      else launch_stream<false>(a, chunk, cpr, items, s, e0, e1);
    }
    return hipGetLastError();
  }
  const unsigned gx = unsigned(max_pos > 0 ? (max_pos + 255) / 256 : 1);
  const dim3 grid(gx, static_cast<unsigned>(rows));
  const size_t shm = size_t(a.H) * a.d * 4 + size_t(a.H) * 4;
  if (a.dt == kBF16)
    launch_k(scan_generic_kernel<uint16_t>, grid, dim3(256), shm, s, e0, e1, a);
  else
    launch_k(scan_generic_kernel<float>, grid, dim3(256), shm, s, e0, e1, a);
  return hipGetLastError();
}

}  // namespace csa
