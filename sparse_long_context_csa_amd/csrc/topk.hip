// Top-K selection, block maxima and the hierarchical candidate pool.
//
// "DeepSeek V4-Flash: The Cost of Deciding What to Read", section "The Lightning Indexer":
// a cheap scoring pass picks the top 512 entries and attention runs over those; section
// "FP4, down to the index scores": the selector decides on FP32 index scores.
// "DeepSeek-V4.1-Flash's KV-Cache Compression, Checked Down to the Byte", section 3, and the
// "DeepSeek-V4.1-Flash" study, "Hierarchical indexing bounds the deeper searches": blocks
// of 8 positions scored by their maximum, at most 2,048 blocks kept as a candidate pool.
//
// Selection rule (exact, integer): candidates are ordered by the 64-bit composite
// (order-preserving key of the fp32 score) << 32 | ~id, so equal scores go to the lower id
// and every composite is distinct. A 1024-thread workgroup holds up to 32,768 candidates
// in registers (wave w owns a contiguous run of 64*ITEMS positions, item j of lane l is
// position w*64*ITEMS + j*64 + l: coalesced loads, and position order is (w, j, l)) and
// runs an MSB-first radix select with 11/11/10-bit digits over LDS histograms, stopping as
// soon as the bucket holding the K-th candidate is taken whole. Selected candidates are
// compacted in position order with wave ballots, so ids come out ascending when positions
// are ascending in id (always the case here). Rows longer than one workgroup's capacity
// are split into segments whose local Top-K candidates are merged by the next level.
#include <limits.h>

#include "csa_common.hpp"
#include "launch.hpp"

namespace csa {

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kBins = 2048;
constexpr int64_t kSegMax = 32768;  // positions per workgroup (ITEMS = 32)

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
};

__device__ __forceinline__ uint32_t digit_of(int level, uint32_t key, int32_t id) {
  const uint32_t v = level < 3 ? key : ~uint32_t(id);
  const int l = level < 3 ? level : level - 3;
  return l == 0 ? (v >> 21) : (l == 1 ? ((v >> 10) & 0x7ffu) : (v & 0x3ffu));
}

// inclusive prefix sum over the block (1024 threads) of v; returns inclusive value
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wtot) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) wtot[wave] = v;
  __syncthreads();
  uint32_t add = 0;
  for (int w = 0; w < wave; ++w) add += wtot[w];
  __syncthreads();
  return v + add;
}

template <int ITEMS>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkLevel L) {
  static_assert(ITEMS <= 64, "items per thread");
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t wtot[kTopkWaves];
  __shared__ uint32_t s_digit, s_above;

  const int64_t r = blockIdx.y;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int64_t cnt = L.count ? int64_t(L.count[r]) : L.count_fixed;
  const int64_t base = int64_t(blockIdx.x) * L.seg;
  const int64_t end = base + L.seg < cnt ? base + L.seg : cnt;
  const int64_t lim = L.id_limit ? int64_t(L.id_limit[r]) : int64_t(INT_MAX);
  const float* sc = L.scores + r * L.s_row;
  const int32_t* ids = L.ids ? L.ids + r * L.i_row : nullptr;

  uint32_t key[ITEMS];
  int32_t id[ITEMS];
  uint64_t valid = 0;
  const int64_t wbase = base + int64_t(wave) * 64 * ITEMS;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const int64_t p = wbase + j * 64 + lane;
    key[j] = 0;
    id[j] = -1;
    if (p < end) {
      const int32_t v = ids ? ids[p] : int32_t(p);
      if (v >= 0 && v < lim) {
        id[j] = v;
        key[j] = order_key(sc[p]);
        valid |= uint64_t(1) << j;
      }
    }
  }
  // number of valid candidates in the segment
  uint32_t nv = __popcll(valid);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nv += __shfl_xor(nv, o);
  if (lane == 0) wtot[wave] = nv;
  __syncthreads();
  uint32_t n = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) n += wtot[w];
  __syncthreads();

  const uint32_t K = uint32_t(L.K);
  uint64_t sel = valid;
  if (n > K) {
    sel = 0;
    uint64_t cand = valid;
    uint32_t need = K;
    bool done = false;
    for (int level = 0; level < 6 && !done; ++level) {
      for (int b = threadIdx.x; b < kBins; b += kTopkThreads) hist[b] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < ITEMS; ++j)
        if ((cand >> j) & 1) atomicAdd(&hist[digit_of(level, key[j], id[j])], 1u);
      __syncthreads();
      // thread t owns bins hi = 2047-2t, lo = 2046-2t (descending order over threads)
      const int hi = kBins - 1 - 2 * int(threadIdx.x), lo = hi - 1;
      const uint32_t h_hi = hist[hi], h_lo = hist[lo];
      const uint32_t incl = block_incl_scan(h_hi + h_lo, wtot);
      const uint32_t excl = incl - h_hi - h_lo;
      if (excl < need && need <= excl + h_hi) { s_digit = hi; s_above = excl; }
      else if (excl + h_hi < need && need <= incl) { s_digit = lo; s_above = excl + h_hi; }
      __syncthreads();
      const uint32_t D = s_digit;
      need -= s_above;
      const uint32_t c = hist[D];
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        if ((cand >> j) & 1) {
          const uint32_t d = digit_of(level, key[j], id[j]);
          if (d > D) sel |= uint64_t(1) << j;
          if (d != D) cand &= ~(uint64_t(1) << j);
        }
      }
      if (c == need) { sel |= cand; done = true; }
      __syncthreads();
    }
    if (!done) {
      // duplicate ids left equal composites: keep the first `need` of them in position order
      uint32_t mine = __popcll(cand);
      uint32_t wc = mine;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) wc += __shfl_xor(wc, o);
      if (lane == 0) wtot[wave] = wc;
      __syncthreads();
      uint32_t before = 0;
      for (int w = 0; w < wave; ++w) before += wtot[w];
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
  if (lane == 0) wtot[wave] = wc;
  __syncthreads();
  uint32_t pos = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    if (w < wave) pos += wtot[w];
    total += wtot[w];
  }
  int32_t* oi = L.o_idx + r * L.o_row + int64_t(blockIdx.x) * L.K;
  float* os = L.o_score ? L.o_score + r * L.o_row + int64_t(blockIdx.x) * L.K : nullptr;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const bool b = (sel >> j) & 1;
    const uint64_t m = __ballot(b);
    if (b) {
      const uint32_t o = pos + uint32_t(lanes_below(m));
      oi[o] = id[j];
      if (os) os[o] = key_to_score(key[j]);
    }
    pos += __popcll(m);
  }
  for (uint32_t k = total + threadIdx.x; k < K; k += kTopkThreads) {
    oi[k] = -1;
    if (os) os[k] = neg_inf();
  }
}

template <int ITEMS>
hipError_t launch_level(const TopkLevel& L, int64_t rows, int64_t nseg, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(nseg), static_cast<unsigned>(rows));
  hipLaunchKernelGGL(topk_kernel<ITEMS>, grid, dim3(kTopkThreads), 0, s, L);
  return hipGetLastError();
}

hipError_t run_level(const TopkLevel& L, int64_t rows, int64_t nseg, hipStream_t s) {
  const int64_t seg = L.seg;
  if (seg <= 1 * kTopkThreads) return launch_level<1>(L, rows, nseg, s);
  if (seg <= 4 * kTopkThreads) return launch_level<4>(L, rows, nseg, s);
  if (seg <= 8 * kTopkThreads) return launch_level<8>(L, rows, nseg, s);
  if (seg <= 16 * kTopkThreads) return launch_level<16>(L, rows, nseg, s);
  return launch_level<32>(L, rows, nseg, s);
}

// Segment plan of one Top-K: level 0 splits max_count positions into segments of at most
// kSegMax; each following level merges the previous level's nseg*K candidates.
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

size_t topk_scratch_bytes(int64_t rows, int64_t max_count, int K) {
  int64_t n = max_count;
  if (n <= kSegMax) return 0;
  int64_t nseg = ceil_div(n, kSegMax);
  // two ping-pong candidate buffers (id + score), sized by the first (largest) level
  const int64_t per = rows * nseg * K;
  return size_t(2 * per * (4 + 4)) + 512;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  int64_t n = a.max_count < 1 ? 1 : a.max_count;
  if (n <= kSegMax) {
    TopkLevel L{a.scores, a.stride, a.ids, a.id_stride, a.id_limit, a.count, n, n, a.K,
                a.out_idx, a.out_score, a.out_stride};
    return run_level(L, a.rows, 1, s);
  }
  int64_t nseg = ceil_div(n, kSegMax);
  const int64_t per = a.rows * nseg * a.K;
  char* base = reinterpret_cast<char*>(a.scratch);
  int32_t* idb[2] = {reinterpret_cast<int32_t*>(base),
                     reinterpret_cast<int32_t*>(base + per * 4)};
  float* scb[2] = {reinterpret_cast<float*>(base + 2 * per * 4),
                   reinterpret_cast<float*>(base + 3 * per * 4)};
  // level 0: segments of the rows
  TopkLevel L0{a.scores, a.stride, a.ids, a.id_stride, a.id_limit, a.count, n, kSegMax, a.K,
               idb[0], scb[0], nseg * a.K};
  hipError_t e = run_level(L0, a.rows, nseg, s);
  if (e != hipSuccess) return e;
  int cur = 0;
  int64_t m = nseg * a.K;   // candidates per row at the current level
  while (true) {
    if (m <= kSegMax) {
      TopkLevel Lf{scb[cur], m, idb[cur], m, nullptr, nullptr, m, m, a.K, a.out_idx,
                   a.out_score, a.out_stride};
      return run_level(Lf, a.rows, 1, s);
    }
    const int64_t ns = ceil_div(m, kSegMax);
    TopkLevel Lm{scb[cur], m, idb[cur], m, nullptr, nullptr, m, kSegMax, a.K, idb[cur ^ 1],
                 scb[cur ^ 1], ns * a.K};
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
                                                        int64_t bstride, int32_t* nb) {
  const int64_t r = blockIdx.y;
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
                            int64_t bmax_stride, int32_t* nb, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t nblk = (max_count + bs - 1) / bs;
  const dim3 grid(unsigned(nblk > 0 ? (nblk + 255) / 256 : 1), unsigned(rows));
  hipLaunchKernelGGL(block_max_kernel, grid, dim3(256), 0, s, scores, stride, count, bs, bmax,
                     bmax_stride, nb);
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
