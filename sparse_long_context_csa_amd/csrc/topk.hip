// Top-K selection, block maxima and the hierarchical candidate pool.
//
// "DeepSeek V4-Flash: The Cost of Deciding What to Read", section "The Lightning Indexer":
// a cheap scoring pass picks the top 512 entries and attention runs over those; section
// "FP4, down to the index scores": the selector decides on FP32 index scores.
// "DeepSeek-V4.1-Flash's KV-Cache Compression, Checked Down to the Byte", section 3, and the
// "DeepSeek-V4.1-Flash" study, "Hierarchical indexing bounds the deeper searches": blocks
// of 8 positions scored by their maximum, at most 2,048 blocks kept as a candidate pool.
//
// Selection rule (exact, integer): candidates are ordered by their order-preserving fp32
// key, then by lower id, i.e. by the 64-bit composite (key << 32 | ~id); every composite is
// distinct. A 512-thread workgroup holds up to 16,384 candidates in registers (wave w owns
// a contiguous run of 64*ITEMS positions, item j of lane l is position w*64*ITEMS + j*64 + l:
// coalesced loads, and position order is (w, j, l)) and runs an MSB-first radix select over
// LDS histograms of 11-bit digits. The first digit starts at the highest bit of
// (key - min key) that the segment can set, so the 2048 bins cover the segment's actual
// score range; selection stops as soon as the bucket holding the K-th candidate is taken
// whole. Selected candidates are compacted in position order with wave ballots, so ids come
// out ascending when positions are ascending in id (always the case here). Rows longer than
// one workgroup's capacity are split into segments; the last segment of a row to finish
// merges the segments' candidates (ticket counter), or further launches do when the
// candidates exceed one workgroup.
#include <limits.h>
#include <stdlib.h>

#include "csa_common.hpp"
#include "launch.hpp"

namespace csa {

namespace {

constexpr int kTopkThreads = 512;   // 8 waves: up to 256 VGPRs per lane, no spills
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kBins = 2048;
constexpr int kBinsPerThread = kBins / kTopkThreads;
constexpr int64_t kSegMax = 16384;   // positions per workgroup (32 per thread)
constexpr int64_t kSegIds = 16384;
constexpr int kMergeItems = 16;      // the fused merge holds up to 16 * 512 candidates

struct TopkLevel {
  const float* scores;
  int64_t s_row;
  const int32_t* ids;    // null: id = position
  int64_t i_row;
  const int32_t* id_limit;
  const int32_t* count;  // null: count_fixed
  int64_t count_fixed;
  int64_t seg;           // positions per segment
  int K;
  int32_t* o_idx;
  float* o_score;        // may be null
  int64_t o_row;         // per-row output stride; segment s writes at + s*K
  // Fused merge: the last segment of a row to finish merges the row's gridDim.x*K
  // candidates (written above) into the final outputs. ticket[r] is zero on entry and is
  // left zero. Null ticket: no merge.
  int32_t* ticket;
  int32_t* f_idx;
  float* f_score;
  int64_t f_row;
};

struct Shared {
  uint32_t hist[kBins];
  uint32_t wred[kTopkWaves][3];
  uint32_t s_digit, s_above, s_last;
};

// inclusive prefix sum over the block of v
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, Shared& sh) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) sh.wred[wave][0] = v;
  __syncthreads();
  uint32_t add = 0;
  for (int w = 0; w < wave; ++w) add += sh.wred[w][0];
  __syncthreads();
  return v + add;
}

// Digit [lo, lo + w) of the composite (kd << 32 | nid), with 32-bit operations only.
__device__ __forceinline__ uint32_t digit_at(uint32_t kd, uint32_t nid, int lo, uint32_t msk) {
  const uint32_t v = lo >= 32 ? (kd >> (lo - 32)) : __builtin_amdgcn_alignbit(kd, nid, lo);
  return v & msk;
}

// Select the Top-K of positions [base, end) of one row; ordered output with -1 padding.
// Requires end - base <= ITEMS * kTopkThreads. Registers per item: the key offset from the
// segment minimum (and the id when ids are explicit).
template <int ITEMS, bool HAS_IDS>
__device__ void select_items(Shared& sh, const float* sc, const int32_t* ids, int64_t base,
                             int64_t end, int64_t lim, uint32_t K, int32_t* oi, float* os) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  uint32_t kd[ITEMS];
  int32_t idv[HAS_IDS ? ITEMS : 1];
  uint64_t valid = 0;
  const int64_t wbase64 = base + int64_t(wave) * 64 * ITEMS;
  const int32_t wbase = int32_t(wbase64);        // positions fit int32 (ids are int32)
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  if (end > base) {
    // batch every load first (addresses clamped into the row), then decode
    float sv[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int64_t p = wbase64 + j * 64 + lane;
      const int64_t pc = p < end ? p : base;
      sv[j] = sc[pc];
      if (HAS_IDS) idv[j] = ids[pc];
    }
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int64_t p = wbase64 + j * 64 + lane;
      const int32_t v = HAS_IDS ? idv[j] : int32_t(p);
      const bool ok = p < end && v >= 0 && v < lim;
      if (HAS_IDS && !ok) idv[j] = -1;
      kd[j] = ok ? order_key(sv[j]) : 0u;
      if (ok) {
        valid |= uint64_t(1) << j;
        kmin = kd[j] < kmin ? kd[j] : kmin;
        kmax = kd[j] > kmax ? kd[j] : kmax;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      kd[j] = 0;
      if (HAS_IDS) idv[j] = -1;
    }
  }
  auto id_of = [&](int j) -> uint32_t {
    if (HAS_IDS) return uint32_t(idv[j]);
    return uint32_t(wbase + j * 64 + lane);
  };
  // block: valid count, key min / max
  uint32_t nv = __popcll(valid);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    nv += __shfl_xor(nv, o);
    const uint32_t a = __shfl_xor(kmin, o), b = __shfl_xor(kmax, o);
    kmin = a < kmin ? a : kmin;
    kmax = b > kmax ? b : kmax;
  }
  if (lane == 0) { sh.wred[wave][0] = nv; sh.wred[wave][1] = kmin; sh.wred[wave][2] = kmax; }
  __syncthreads();
  uint32_t n = 0;
  kmin = 0xffffffffu;
  kmax = 0u;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    n += sh.wred[w][0];
    kmin = sh.wred[w][1] < kmin ? sh.wred[w][1] : kmin;
    kmax = sh.wred[w][2] > kmax ? sh.wred[w][2] : kmax;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) kd[j] -= kmin;   // valid items: key - kmin

  uint64_t sel = valid;
  if (n > K) {
    sel = 0;
    uint64_t cand = valid;
    uint32_t need = K;
    bool done = false;
    const uint32_t range = kmax - kmin;
    const int bl = range ? 32 - __clz(range) : 0;
    int hi = bl ? 31 + bl : 31;   // highest bit any composite (key - kmin) << 32 | ~id can set
    while (!done && hi >= 0) {
      const int w = hi + 1 < 11 ? hi + 1 : 11;
      const int lo = hi + 1 - w;
      const uint32_t msk = (1u << w) - 1u;
      for (int b = threadIdx.x; b < kBins; b += kTopkThreads) sh.hist[b] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < ITEMS; ++j)
        if ((cand >> j) & 1) atomicAdd(&sh.hist[digit_at(kd[j], ~id_of(j), lo, msk)], 1u);
      __syncthreads();
      // thread t owns bins 2047-4t .. 2044-4t (descending order over threads)
      const int btop = kBins - 1 - kBinsPerThread * int(threadIdx.x);
      uint32_t hb[kBinsPerThread], loc = 0;
#pragma unroll
      for (int q = 0; q < kBinsPerThread; ++q) { hb[q] = sh.hist[btop - q]; loc += hb[q]; }
      const uint32_t incl = block_incl_scan(loc, sh);
      uint32_t above = incl - loc;
#pragma unroll
      for (int q = 0; q < kBinsPerThread; ++q) {
        if (above < need && need <= above + hb[q]) { sh.s_digit = btop - q; sh.s_above = above; }
        above += hb[q];
      }
      __syncthreads();
      const uint32_t D = sh.s_digit;
      need -= sh.s_above;
      const uint32_t c = sh.hist[D];
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        if ((cand >> j) & 1) {
          const uint32_t d = digit_at(kd[j], ~id_of(j), lo, msk);
          if (d > D) sel |= uint64_t(1) << j;
          if (d != D) cand &= ~(uint64_t(1) << j);
        }
      }
      if (c == need) { sel |= cand; done = true; }
      hi = lo - 1;
      __syncthreads();
    }
    if (!done) {
      // duplicate ids left equal composites: keep the first `need` of them in position order
      uint32_t wc = __popcll(cand);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) wc += __shfl_xor(wc, o);
      if (lane == 0) sh.wred[wave][0] = wc;
      __syncthreads();
      uint32_t before = 0;
      for (int w2 = 0; w2 < wave; ++w2) before += sh.wred[w2][0];
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        const bool b = (cand >> j) & 1;
        const uint64_t m = __ballot(b);
        if (b && before + uint32_t(lanes_below(m)) < need) sel |= uint64_t(1) << j;
        before += __popcll(m);
      }
      __syncthreads();
    }
  }

  // ordered compaction of the selected candidates
  uint32_t wc = __popcll(sel);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) wc += __shfl_xor(wc, o);
  if (lane == 0) sh.wred[wave][0] = wc;
  __syncthreads();
  uint32_t pos = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    if (w < wave) pos += sh.wred[w][0];
    total += sh.wred[w][0];
  }
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const bool b = (sel >> j) & 1;
    const uint64_t m = __ballot(b);
    if (b) {
      const uint32_t o = pos + uint32_t(lanes_below(m));
      oi[o] = int32_t(id_of(j));
      if (os) os[o] = key_to_score(kd[j] + kmin);
    }
    pos += __popcll(m);
  }
  for (uint32_t k = total + threadIdx.x; k < K; k += kTopkThreads) {
    oi[k] = -1;
    if (os) os[k] = neg_inf();
  }
  __syncthreads();
}

template <int ITEMS, bool HAS_IDS>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkLevel L) {
  __shared__ Shared sh;
  const int64_t r = blockIdx.y;
  const int64_t cnt = L.count ? int64_t(L.count[r]) : L.count_fixed;
  const int64_t base = int64_t(blockIdx.x) * L.seg;
  const int64_t end = base + L.seg < cnt ? base + L.seg : cnt;
  const int64_t lim = L.id_limit ? int64_t(L.id_limit[r]) : int64_t(INT_MAX);
  int32_t* oi = L.o_idx + r * L.o_row + int64_t(blockIdx.x) * L.K;
  float* os = L.o_score ? L.o_score + r * L.o_row + int64_t(blockIdx.x) * L.K : nullptr;
  select_items<ITEMS, HAS_IDS>(sh, L.scores + r * L.s_row,
                               HAS_IDS ? L.ids + r * L.i_row : nullptr, base, end, lim,
                               uint32_t(L.K), oi, os);
  if (L.ticket == nullptr) return;
  // the last segment of the row to finish merges every segment's candidates
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int32_t t = atomicAdd(&L.ticket[r], 1);
    sh.s_last = (t == int32_t(gridDim.x) - 1);
  }
  __syncthreads();
  if (!sh.s_last) return;
  __threadfence();
  const int64_t m = int64_t(gridDim.x) * L.K;
  select_items<kMergeItems, true>(sh, L.o_score + r * L.o_row, L.o_idx + r * L.o_row, 0, m,
                                  int64_t(INT_MAX), uint32_t(L.K), L.f_idx + r * L.f_row,
                                  L.f_score ? L.f_score + r * L.f_row : nullptr);
  if (threadIdx.x == 0) L.ticket[r] = 0;
}

template <int ITEMS, bool HAS_IDS>
hipError_t launch_level(const TopkLevel& L, int64_t rows, int64_t nseg, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(nseg), static_cast<unsigned>(rows));
  hipLaunchKernelGGL((topk_kernel<ITEMS, HAS_IDS>), grid, dim3(kTopkThreads), 0, s, L);
  return hipGetLastError();
}

template <bool HAS_IDS>
hipError_t run_level_t(const TopkLevel& L, int64_t rows, int64_t nseg, hipStream_t s) {
  const int64_t seg = L.seg;
  if (seg <= 1 * kTopkThreads) return launch_level<1, HAS_IDS>(L, rows, nseg, s);
  if (seg <= 4 * kTopkThreads) return launch_level<4, HAS_IDS>(L, rows, nseg, s);
  if (seg <= 8 * kTopkThreads) return launch_level<8, HAS_IDS>(L, rows, nseg, s);
  if (seg <= 16 * kTopkThreads) return launch_level<16, HAS_IDS>(L, rows, nseg, s);
  return launch_level<32, HAS_IDS>(L, rows, nseg, s);
}

hipError_t run_level(const TopkLevel& L, int64_t rows, int64_t nseg, hipStream_t s) {
  return L.ids ? run_level_t<true>(L, rows, nseg, s) : run_level_t<false>(L, rows, nseg, s);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return v ? atoi(v) : dflt;
}
// Tuning overrides (read once): positions per segment and whether the merge is fused.
int64_t tune_seg() {
  static const int64_t v = [] {
    int64_t x = env_int("CSA_TUNE_TOPK_SEG", int(kSegMax));
    return x >= 512 && x <= kSegMax ? (x + 511) / 512 * 512 : kSegMax;
  }();
  return v;
}
bool tune_fuse() {
  static const bool v = env_int("CSA_TUNE_TOPK_FUSE", 0) != 0;
  return v;
}

int64_t seg_of(bool has_ids) { return has_ids ? kSegIds : tune_seg(); }

// Scratch layout: two ping-pong candidate buffers (ids, scores) sized by the first level,
// then one merge ticket per row.
struct Plan {
  int64_t seg, nseg, per;
  size_t ticket_off, bytes;
};
Plan plan(int64_t rows, int64_t n, int K, bool has_ids) {
  Plan p{};
  p.seg = seg_of(has_ids);
  if (n <= p.seg) return p;
  p.nseg = ceil_div(n, p.seg);
  p.per = rows * p.nseg * K;
  p.ticket_off = size_t(4 * p.per * 4);
  p.bytes = p.ticket_off + size_t(rows) * 4;
  return p;
}

}  // namespace

size_t topk_scratch_bytes(int64_t rows, int64_t max_count, int K) {
  const Plan a = plan(rows, max_count, K, true), b = plan(rows, max_count, K, false);
  return a.bytes > b.bytes ? a.bytes : b.bytes;
}

int32_t* topk_ticket(void* scratch, int64_t rows, int64_t max_count, int K, bool has_ids) {
  const Plan p = plan(rows, max_count, K, has_ids);
  if (p.bytes == 0 || scratch == nullptr) return nullptr;
  return reinterpret_cast<int32_t*>(reinterpret_cast<char*>(scratch) + p.ticket_off);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  const bool has_ids = a.ids != nullptr;
  const int64_t n = a.max_count < 1 ? 1 : a.max_count;
  const Plan p = plan(a.rows, n, a.K, has_ids);
  if (p.bytes == 0) {
    TopkLevel L{a.scores, a.stride, a.ids, a.id_stride, a.id_limit, a.count, n, n, a.K,
                a.out_idx, a.out_score, a.out_stride, nullptr, nullptr, nullptr, 0};
    return run_level(L, a.rows, 1, s);
  }
  char* base = reinterpret_cast<char*>(a.scratch);
  int32_t* idb[2] = {reinterpret_cast<int32_t*>(base),
                     reinterpret_cast<int32_t*>(base + p.per * 4)};
  float* scb[2] = {reinterpret_cast<float*>(base + 2 * p.per * 4),
                   reinterpret_cast<float*>(base + 3 * p.per * 4)};
  int32_t* ticket = reinterpret_cast<int32_t*>(base + p.ticket_off);
  const bool fuse = tune_fuse() && a.tickets_zeroed &&
                    p.nseg * a.K <= int64_t(kMergeItems) * kTopkThreads;
  // level 0: segments of the rows (+ the fused merge)
  TopkLevel L0{a.scores, a.stride, a.ids, a.id_stride, a.id_limit, a.count, n, p.seg, a.K,
               idb[0], scb[0], p.nseg * a.K, fuse ? ticket : nullptr, a.out_idx, a.out_score,
               a.out_stride};
  hipError_t e = run_level(L0, a.rows, p.nseg, s);
  if (e != hipSuccess || fuse) return e;
  int cur = 0;
  int64_t m = p.nseg * a.K;   // candidates per row at the current level
  while (true) {
    if (m <= kSegIds) {
      TopkLevel Lf{scb[cur], m, idb[cur], m, nullptr, nullptr, m, m, a.K, a.out_idx,
                   a.out_score, a.out_stride, nullptr, nullptr, nullptr, 0};
      return run_level(Lf, a.rows, 1, s);
    }
    const int64_t ns = ceil_div(m, kSegIds);
    TopkLevel Lm{scb[cur], m, idb[cur], m, nullptr, nullptr, m, kSegIds, a.K, idb[cur ^ 1],
                 scb[cur ^ 1], ns * a.K, nullptr, nullptr, nullptr, 0};
    e = run_level(Lm, a.rows, ns, s);
    if (e != hipSuccess) return e;
    cur ^= 1;
    m = ns * a.K;
  }
}

// ---- block maxima ------------------------------------------------------------------------
__global__ __launch_bounds__(256) void block_max_kernel(const float* __restrict__ scores,
                                                        int64_t stride,
                                                        const int32_t* __restrict__ count,
                                                        int bs, float* __restrict__ bmax,
                                                        int64_t bstride, int32_t* nb,
                                                        int32_t* zero, int64_t n_zero) {
  const int64_t r = blockIdx.y;
  if (zero && blockIdx.x == 0 && r == 0)
    for (int64_t i = threadIdx.x; i < n_zero; i += blockDim.x) zero[i] = 0;
  const int64_t n = count[r];
  const int64_t nblk = (n + bs - 1) / bs;
  if (blockIdx.x == 0 && threadIdx.x == 0) nb[r] = int32_t(nblk);
  const int64_t b = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (b >= nblk) return;
  const float* sr = scores + r * stride;
  const int64_t e0 = b * bs;
  const int64_t e1 = e0 + bs < n ? e0 + bs : n;
  float mx = sr[e0];
  for (int64_t e = e0 + 1; e < e1; ++e) mx = fmaxf(mx, sr[e]);
  bmax[r * bstride + b] = mx;
}

hipError_t launch_block_max(const float* scores, int64_t stride, const int32_t* count,
                            int64_t rows, int64_t max_count, int bs, float* bmax,
                            int64_t bmax_stride, int32_t* nb, int32_t* zero, int64_t n_zero,
                            hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t nblk = (max_count + bs - 1) / bs;
  const dim3 grid(unsigned(nblk > 0 ? (nblk + 255) / 256 : 1), unsigned(rows));
  hipLaunchKernelGGL(block_max_kernel, grid, dim3(256), 0, s, scores, stride, count, bs, bmax,
                     bmax_stride, nb, zero, n_zero);
  return hipGetLastError();
}

// ---- pool of the selected blocks ---------------------------------------------------------
// blocks[r] holds ascending block ids (-1 padded); only the block holding the last visible
// entry can be partial and, being the highest id, it comes last, so the pool is a compact
// ascending prefix followed by -1.
__global__ __launch_bounds__(256) void pool_build_kernel(const int32_t* __restrict__ blocks,
                                                         int max_blocks, int bs,
                                                         const int32_t* __restrict__ n_vis,
                                                         int32_t* __restrict__ pool) {
  const int64_t r = blockIdx.y;
  const int64_t k = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t n = int64_t(max_blocks) * bs;
  if (k >= n) return;
  const int32_t b = blocks[r * max_blocks + k / bs];
  const int64_t e = int64_t(b) * bs + k % bs;
  pool[r * n + k] = (b >= 0 && e < n_vis[r]) ? int32_t(e) : -1;
}

hipError_t launch_pool_build(const int32_t* blocks, int64_t rows, int max_blocks, int bs,
                             const int32_t* n_vis, int32_t* pool, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t n = int64_t(max_blocks) * bs;
  const dim3 grid(unsigned((n + 255) / 256), unsigned(rows));
  hipLaunchKernelGGL(pool_build_kernel, grid, dim3(256), 0, s, blocks, max_blocks, bs, n_vis,
                     pool);
  return hipGetLastError();
}

// ---- scores_all export -------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_scores_kernel(const float* __restrict__ scores,
                                                          int64_t stride,
                                                          const int32_t* __restrict__ count,
                                                          int64_t n_keys, float* __restrict__ out) {
  const int64_t r = blockIdx.y;
  const int64_t p = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (p >= n_keys) return;
  out[r * n_keys + p] = p < count[r] ? scores[r * stride + p] : neg_inf();
}

hipError_t launch_fill_scores(const float* scores, int64_t stride, const int32_t* count,
                              int64_t rows, int64_t n_keys, float* out, hipStream_t s) {
  if (rows == 0 || n_keys == 0) return hipSuccess;
  const dim3 grid(unsigned((n_keys + 255) / 256), unsigned(rows));
  hipLaunchKernelGGL(fill_scores_kernel, grid, dim3(256), 0, s, scores, stride, count, n_keys,
                     out);
  return hipGetLastError();
}

}  // namespace csa
