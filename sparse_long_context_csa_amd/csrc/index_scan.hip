// Lightning-indexer scan: I(t,s) = sum_h w(t,h) * ReLU(q_I(t,h) . K_s) for every candidate.
//
// "DeepSeek V4-Flash: The Cost of Deciding What to Read", section "The Lightning Indexer":
// 64 indexer heads of dim 128 per query, one compressed indexer key per entry, a rectified
// dot product per head, summed with the per-head gate w; section "The indexer is O(n), and
// that is the ceiling": the scan touches every visible entry and never becomes sparse.
//
// Three kernels:
//  * scan_decode_kernel (bf16, 64 heads x 128): few query rows, many keys. The contraction
//    is a [64 heads x 128] x [128 x 16 keys] MFMA (v_mfma_f32_16x16x32_bf16) per tile; the
//    query stays in VGPRs as the A operand and every key row is read once from HBM straight
//    into the B operand (no LDS: nothing is reused across waves). The channel order inside
//    each MFMA is permuted so a lane reads 64 contiguous bytes of its key row. ReLU, gate
//    and head sum run on the accumulator lanes, two xor-shuffles finish the head sum.
//  * scan_prefill_kernel (bf16, 64 x 128): many query rows (a prefill chunk). 8 query rows
//    per workgroup (one per wave, A operand in VGPRs); 64-key tiles are staged in LDS once
//    and reused by the 8 waves, double-buffered with the next tile's global loads.
//  * scan_generic_kernel: any head count/dim and fp32; one thread per candidate.
// Visibility: entry i is usable by a query at t only if m*(i+1)-1 <= t ("The sliding window
// is not an optimisation"); positions past a row's visible count are never scored.
#include <stdlib.h>

#include "csa_common.hpp"
#include "ingest.hpp"
#include "launch.hpp"

namespace csa {

namespace {

constexpr int kIH = 64;    // indexer heads on the MFMA paths
constexpr int kID = 128;   // indexer dim on the MFMA paths

__device__ __forceinline__ int64_t row_visible(const ScanArgs& a, int64_t r) {
  const int64_t sq = r / a.n_q;
  int64_t cap = a.e_cap;
  if (a.e_count) {
    const int64_t ec = a.e_count[sq];
    cap = ec < cap ? (ec < 0 ? 0 : ec) : cap;
  }
  return visible_entries(a.q_pos[r], a.m, cap);
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
    for (int i = 0; i < 4; ++i) part = fmaf(wv[mt][i], fmaxf(acc[mt][i], 0.f), part);
  part += __shfl_xor(part, 16);
  part += __shfl_xor(part, 32);
  return part;
}

// maximum over the 16 lanes of this lane's group (lanes 16j .. 16j+15 hold one key tile)
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  return v;
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

// Pool the new entry's indexer key from the values a lane holds (channels 2*lane and
// 2*lane+1 of m rows, the new row in `slot`), store it to the cache, and when `mine` put it
// into this lane's B operand: channels ks*32 + g*8 .. +8 come from lanes ks*16 + g*4 + 0..3.
constexpr int kFuseM = 8;   // entries of up to 8 rows are pooled this way
__device__ __forceinline__ void fuse_new_key(const IngestArgs& ig, int64_t r, int64_t e, int slot,
                                             int lane, int g, bool mine, uint32_t xn, uint32_t zn,
                                             const uint32_t (&xt)[kFuseM],
                                             const uint32_t (&zt)[kFuseM],
                                             const uint32_t (&bb)[kFuseM], bf16x8_t (&B)[4]) {
  const int m = ig.m;
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
        av[j] = half(j == slot ? zn : zt[j]) + half(bb[j]);
        mx = fmaxf(mx, av[j]);
      }
    }
    float sum = 0.f, acc = 0.f;
#pragma unroll
    for (int j = 0; j < kFuseM; ++j)
      if (j < m) {
        const float ex = expf(av[j] - mx);
        sum += ex;
        acc = fmaf(ex, half(j == slot ? xn : xt[j]), acc);
      }
    res[h] = acc / sum;
  }
  const uint32_t pk = uint32_t(f32_to_bf16(res[0])) | (uint32_t(f32_to_bf16(res[1])) << 16);
  reinterpret_cast<uint32_t*>(ig.k_idx)[(r * ig.e_cap + e) * (kID / 2) + lane] = pk;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint32_t wds[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) wds[k] = uint32_t(__shfl(int(pk), ks * 16 + g * 4 + k));
    if (mine) B[ks] = *reinterpret_cast<const bf16x8_t*>(wds);
  }
}

}  // namespace

// Persistent grid: work item it = (row, chunk) = (it / cpr, it % cpr), chunk positions
// [c*chunk, (c+1)*chunk); blocks stride over the items, so the grid is sized to the machine
// rather than to the work (no partially filled last wave of blocks). Within an item, wave w
// scores 16-key tiles w, w+4, ... and keeps PF further tiles of keys in flight (registers)
// while the MFMAs of the current tile run.
template <bool kCand, int PF, bool NT>
__global__ __launch_bounds__(256) void scan_decode_kernel(ScanArgs a, int chunk, int64_t cpr,
                                                          int64_t n_items) {
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
    float* gmax = a.gmax + r * a.gmax_stride;
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
    // Decode ingest folded in: the entry that the step's token completes is pooled by the
    // wave that scores it. Its inputs (2 channels per lane) load now, the pooling runs at
    // that tile, and lane shuffles place the key in the B operand of its column.
    int64_t e_new = -1;
    int slot = 0;
    uint32_t pxn = 0, pzn = 0, pxt[kFuseM], pzt[kFuseM], pb[kFuseM];
#pragma unroll
    for (int j = 0; j < kFuseM; ++j) pxt[j] = pzt[j] = pb[j] = 0u;
    if (fuse) {
      const int64_t t = a.ingest.pos[r];
      const int64_t e = (t + 1) / a.ingest.m - 1;
      if (t >= 0 && (t + 1) % a.ingest.m == 0 && e >= c0 && e < c1 &&
          int((e - c0) >> 4) % 4 == wave) {
        e_new = e;
        slot = int(t % a.ingest.m);
        const IngestArgs& ig = a.ingest;
        const int m = ig.m;
        pxn = reinterpret_cast<const uint32_t*>(ig.xi_new)[r * (kID / 2) + lane];
        pzn = reinterpret_cast<const uint32_t*>(ig.zi_new)[r * (kID / 2) + lane];
#pragma unroll
        for (int j = 0; j < kFuseM; ++j) {
          if (j < m && j != slot) {
            pxt[j] = reinterpret_cast<const uint32_t*>(ig.xi_tail)[(r * m + j) * (kID / 2) + lane];
            pzt[j] = reinterpret_cast<const uint32_t*>(ig.zi_tail)[(r * m + j) * (kID / 2) + lane];
          }
          if (j < m) pb[j] = reinterpret_cast<const uint32_t*>(ig.bias_i)[j * (kID / 2) + lane];
        }
      }
    }
    const int64_t t0 = c0 + wave * 16;
    if (t0 >= c1) continue;
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
            fuse_new_key(a.ingest, r, e_new, slot, lane, g, col == int(e_new - tl), pxn, pzn, pxt,
                         pzt, pb, buf[u]);
          const float s = tile_score(A, buf[u], wv);
          const int64_t p = tl + col;
          const float sv = (p < c1 && ok[u]) ? s : neg_inf();
          if (g == 0 && p < c1) out[p] = sv;
          const float gm = max16(sv);
          if (lane == 0) gmax[tl >> 4] = gm;
          const int64_t nx = tl + int64_t(PF + 1) * 64;
          if (nx < c1) load_key_B<NT>(kb + key_row(nx + col, ok[u]) * kID, g, buf[u]);
        } else {
          more = false;
        }
      }
    }
  }
}

// ---- prefill: 8 query rows per block, 64-key tiles staged through LDS ----------------------
constexpr int kPQ = 8;            // query rows per block (one per wave)
constexpr int kPT = 64;           // keys per tile
constexpr int kPRow = 272;        // LDS bytes per key row (256 + 16 pad: conflict-free b128)

__global__ __launch_bounds__(512) void scan_prefill_kernel(ScanArgs a, int keys_per_block) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][kPT * kPRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int64_t rows = a.n_seq * a.n_q;
  // query rows of this block: kPQ consecutive rows of one sequence
  const int64_t groups_per_seq = (a.n_q + kPQ - 1) / kPQ;
  const int64_t sq = blockIdx.y / groups_per_seq;
  const int64_t i0 = (blockIdx.y % groups_per_seq) * kPQ;
  const int64_t qi = i0 + wave;
  const bool row_ok = qi < a.n_q;
  const int64_t r = sq * a.n_q + (row_ok ? qi : i0);
  const int64_t n_vis = row_ok ? row_visible(a, r) : 0;
  if (row_ok && blockIdx.x == 0 && lane == 0) {
    a.n_vis[r] = int32_t(n_vis);
    a.count[r] = int32_t(n_vis);
  }
  // block-wide extent: the largest visible count among the block's rows
  __shared__ int64_t s_nmax[kPQ];
  if (lane == 0) s_nmax[wave] = n_vis;
  __syncthreads();
  int64_t nmax = 0;
#pragma unroll
  for (int i = 0; i < kPQ; ++i) nmax = s_nmax[i] > nmax ? s_nmax[i] : nmax;
  const int64_t k0 = int64_t(blockIdx.x) * keys_per_block;
  const int64_t k1 = k0 + keys_per_block < nmax ? k0 + keys_per_block : nmax;
  if (k0 >= k1) return;
  (void)rows;

  bf16x8_t A[4][4];
  load_query_A(reinterpret_cast<const uint16_t*>(a.q) + r * kIH * kID, lane, A);
  float wv[4][4];
  load_gates(a.w + r * kIH, lane, wv);
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.keys) + sq * a.e_cap * kID;
  float* out = a.scores + r * a.score_stride;
  float* gmax = a.gmax + r * a.gmax_stride;

  // cooperative tile load: thread t moves 16-byte chunks t and t+512 of the 64x256 B tile
  const int ch0 = threadIdx.x, ch1 = threadIdx.x + 512;
  auto gload = [&](int64_t base, bf16x8_t& v0, bf16x8_t& v1) {
    const int64_t r0 = base + (ch0 >> 4), r1 = base + (ch1 >> 4);
    const int64_t s0 = r0 < k1 ? r0 : k1 - 1, s1 = r1 < k1 ? r1 : k1 - 1;
    v0 = __builtin_nontemporal_load(reinterpret_cast<const bf16x8_t*>(kb + s0 * kID) + (ch0 & 15));
    v1 = __builtin_nontemporal_load(reinterpret_cast<const bf16x8_t*>(kb + s1 * kID) + (ch1 & 15));
  };
  auto lstore = [&](int buf, const bf16x8_t& v0, const bf16x8_t& v1) {
    *reinterpret_cast<bf16x8_t*>(&lds[buf][(ch0 >> 4) * kPRow + (ch0 & 15) * 16]) = v0;
    *reinterpret_cast<bf16x8_t*>(&lds[buf][(ch1 >> 4) * kPRow + (ch1 & 15) * 16]) = v1;
  };

  bf16x8_t v0, v1;
  gload(k0, v0, v1);
  lstore(0, v0, v1);
  __syncthreads();
  int buf = 0;
  for (int64_t base = k0; base < k1; base += kPT) {
    const bool more = base + kPT < k1;
    if (more) gload(base + kPT, v0, v1);
    if (base < n_vis) {
      const unsigned char* tb = lds[buf];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        bf16x8_t B[4];
        const unsigned char* rp = tb + (nt * 16 + col) * kPRow + g * 16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) B[ks] = *reinterpret_cast<const bf16x8_t*>(rp + ks * 64);
        const float s = tile_score(A, B, wv);
        const int64_t p = base + nt * 16 + col;
        if (g == 0 && p < n_vis) out[p] = s;
        const float gm = max16(p < n_vis ? s : neg_inf());
        if (lane == 0) gmax[(base + nt * 16) >> 4] = gm;
      }
    }
    if (more) {
      lstore(buf ^ 1, v0, v1);
      __syncthreads();
      buf ^= 1;
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
  const float gm = max16(s);
  if ((threadIdx.x & 15) == 0 && live) a.gmax[r * a.gmax_stride + (p >> 4)] = gm;
}

static bool fast_shape(const ScanArgs& a) { return a.dt == kBF16 && a.H == kIH && a.d == kID; }

// Decode-scan launch shape: positions per work item, key tiles in flight per wave beyond the
// current one, and blocks resident per CU (the persistent grid is n_cu * blocks_per_cu).
struct ScanTune {
  int chunk = 2048, pf = 1, blocks_per_cu = 2, nt = 1;
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

template <bool kCand, int PF, bool NT>
static void launch_decode(const ScanArgs& a, int64_t rows, int64_t max_pos, hipStream_t s) {
  const ScanTune& t = scan_tune();
  const int bpc = t.blocks_per_cu > 0 ? t.blocks_per_cu : 2;
  int64_t grid = int64_t(n_cu()) * bpc;
  // chunk: the tuned size, shrunk (to >= 256 positions) until there is at least one work
  // item per resident block
  int chunk = t.chunk > 0 ? (t.chunk + 63) / 64 * 64 : 2048;
  while (chunk > 256 && rows * ((max_pos + chunk - 1) / chunk) < grid) chunk /= 2;
  chunk = (chunk + 63) / 64 * 64;
  const int64_t cpr = max_pos > 0 ? (max_pos + chunk - 1) / chunk : 1;
  const int64_t items = rows * cpr;
  if (grid > items) grid = items;
  hipLaunchKernelGGL((scan_decode_kernel<kCand, PF, NT>), dim3(static_cast<unsigned>(grid)),
                     dim3(256), 0, s, a, chunk, cpr, items);
}

template <bool kCand>
static void launch_decode_pf(const ScanArgs& a, int64_t rows, int64_t max_pos, hipStream_t s) {
  const bool nt = scan_tune().nt != 0;
  switch (scan_tune().pf) {
    case 1: nt ? launch_decode<kCand, 1, true>(a, rows, max_pos, s)
               : launch_decode<kCand, 1, false>(a, rows, max_pos, s); break;
    case 3: nt ? launch_decode<kCand, 3, true>(a, rows, max_pos, s)
               : launch_decode<kCand, 3, false>(a, rows, max_pos, s); break;
    default: nt ? launch_decode<kCand, 2, true>(a, rows, max_pos, s)
                : launch_decode<kCand, 2, false>(a, rows, max_pos, s); break;
  }
}

bool scan_fuses_ingest(int dt, int H, int d, int m) {
  return dt == kBF16 && H == kIH && d == kID && m <= kFuseM;
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t s) {
  const int64_t rows = a.n_seq * a.n_q;
  if (rows == 0) return hipSuccess;
  const int64_t max_pos = a.cand ? a.n_cand : a.e_cap;
  if (fast_shape(a) && a.cand == nullptr && a.n_q >= 16) {
    const int keys_per_block = 4096;
    const int64_t groups = a.n_seq * ((a.n_q + kPQ - 1) / kPQ);
    const dim3 grid(static_cast<unsigned>((a.e_cap + keys_per_block - 1) / keys_per_block),
                    static_cast<unsigned>(groups));
    hipLaunchKernelGGL(scan_prefill_kernel, grid, dim3(512), 0, s, a, keys_per_block);
    return hipGetLastError();
  }
  if (fast_shape(a)) {
    if (a.cand) launch_decode_pf<true>(a, rows, max_pos, s);
    else launch_decode_pf<false>(a, rows, max_pos, s);
    return hipGetLastError();
  }
  const unsigned gx = unsigned(max_pos > 0 ? (max_pos + 255) / 256 : 1);
  const dim3 grid(gx, static_cast<unsigned>(rows));
  const size_t shm = size_t(a.H) * a.d * 4 + size_t(a.H) * 4;
  if (a.dt == kBF16)
    hipLaunchKernelGGL(scan_generic_kernel<uint16_t>, grid, dim3(256), shm, s, a);
  else
    hipLaunchKernelGGL(scan_generic_kernel<float>, grid, dim3(256), shm, s, a);
  return hipGetLastError();
}

}  // namespace csa
