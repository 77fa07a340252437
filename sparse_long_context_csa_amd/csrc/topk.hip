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
// one workgroup's capacity are split into segments whose local Top-K candidates are merged
// by further launches.
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
constexpr int64_t kSegMax = 16384;   // positions per workgroup, implicit ids

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

// A thread's run of ITEMS consecutive positions sits at LDS words [t*(ITEMS+4), +ITEMS): the
// 4-word pad makes the 16-byte reads of 16 consecutive lanes hit 64 distinct banks.
constexpr int kMaxItems = 32;          // implicit ids: 16,384 positions per workgroup
constexpr int kMaxItemsIds = 16;       // explicit ids: 8,192 (two padded arrays must fit)

constexpr int kListCap = 8192;         // candidate list (position order) of the sampled path
constexpr int kListPerThread = kListCap / kTopkThreads;

template <bool HAS_IDS>
struct Shared {
  static constexpr int kRun = (HAS_IDS ? kMaxItemsIds : kMaxItems) + 4;
  uint32_t hist[kBins];
  uint32_t wred[kTopkWaves][3];
  uint32_t s_digit, s_above, s_last;
  alignas(16) uint32_t key[kTopkThreads * kRun];            // order keys, padded runs
  alignas(16) int32_t id[HAS_IDS ? kTopkThreads * kRun : 4]; // explicit ids, padded runs
  // candidate list (key - kmin, ~id); its first K slots also stage the ordered output
  alignas(16) uint32_t lkd[kListCap];
  alignas(16) uint32_t lnid[kListCap];
};

// exclusive prefix sum over the block of v; *total receives the block sum
template <typename SH>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, SH& sh, uint32_t* total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(x, o);
    if (lane >= o) x += u;
  }
  if (lane == 63) sh.wred[wave][0] = x;
  __syncthreads();
  uint32_t add = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const uint32_t t = sh.wred[w][0];
    if (w < wave) add += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return x - v + add;
}

template <typename SH>
__device__ __forceinline__ uint32_t block_sum(uint32_t v, SH& sh) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if (lane == 0) sh.wred[wave][0] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) t += sh.wred[w][0];
  __syncthreads();
  return t;
}

// Digit [lo, lo + w) of the composite (kd << 32 | nid), with 32-bit operations only.
__device__ __forceinline__ uint32_t digit_at(uint32_t kd, uint32_t nid, int lo, uint32_t msk) {
  const uint32_t v = lo >= 32 ? (kd >> (lo - 32)) : __builtin_amdgcn_alignbit(kd, nid, lo);
  return v & msk;
}
// (kd << 32 | nid) >> lo as 64 bits
__device__ __forceinline__ uint64_t prefix_at(uint32_t kd, uint32_t nid, int lo) {
  const uint64_t u = (uint64_t(kd) << 32) | nid;
  return lo >= 64 ? 0 : (u >> lo);
}

// Bin (of the histogram just built) holding the need-th largest: thread t owns bins
// 2047-4t .. 2044-4t (descending over threads). Sets sh.s_digit / sh.s_above.
template <typename SH>
__device__ __forceinline__ void find_bin(SH& sh, uint32_t need) {
  const int btop = kBins - 1 - kBinsPerThread * int(threadIdx.x);
  uint32_t hb[kBinsPerThread], loc = 0;
#pragma unroll
  for (int q = 0; q < kBinsPerThread; ++q) { hb[q] = sh.hist[btop - q]; loc += hb[q]; }
  uint32_t tot;
  uint32_t above = block_excl_scan(loc, sh, &tot);
#pragma unroll
  for (int q = 0; q < kBinsPerThread; ++q) {
    if (above < need && need <= above + hb[q]) { sh.s_digit = btop - q; sh.s_above = above; }
    above += hb[q];
  }
  __syncthreads();
}

struct Thresh {
  int lo;          // selected: composite >> lo  >  P, or == P (all when done)
  uint64_t P;
  uint32_t need;   // when !done: how many of the items equal to P are taken (lowest positions)
  bool done;
};

// Select the Top-K of positions [base, end) of one row; ordered output with -1 padding.
// The segment lives in LDS in position order; thread t owns positions t*ITEMS .. +ITEMS,
// so per-thread masks (32-bit) track validity, candidacy and selection, and the ordered
// compaction is one block scan of per-thread counts.
// Requires end - base <= ITEMS * kTopkThreads, ITEMS in {4, 8, 16, 32}, K <= 2048.
template <int ITEMS, bool HAS_IDS>
__device__ void select_items(Shared<HAS_IDS>& sh, const float* sc, const int32_t* ids,
                             int64_t base, int64_t end, int64_t lim, uint32_t K, int32_t* oi,
                             float* os) {
  static_assert(ITEMS % 4 == 0 && ITEMS <= (HAS_IDS ? kMaxItemsIds : kMaxItems), "items");
  constexpr int RUN = ITEMS + 4;                 // padded run stride (words)
  const int tid = threadIdx.x;
  const int64_t nseg = end > base ? end - base : 0;
  // 1. coalesced copy of the segment into LDS: 16-byte loads of 4 positions (same run)
  for (int q = 0; q < ITEMS / 4; ++q) {
    const int i0 = 4 * (tid + kTopkThreads * q);
    if (i0 >= nseg) continue;
    const int l0 = (i0 / ITEMS) * RUN + (i0 % ITEMS);
    if (i0 + 3 < nseg) {
      const float4 v = *reinterpret_cast<const float4*>(sc + base + i0);
      *reinterpret_cast<uint4*>(&sh.key[l0]) =
          make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                     __float_as_uint(v.w));
      if (HAS_IDS) {
        // ids are caller memory: element loads (no read past the row)
        int4 iv;
        iv.x = ids[base + i0]; iv.y = ids[base + i0 + 1];
        iv.z = ids[base + i0 + 2]; iv.w = ids[base + i0 + 3];
        *reinterpret_cast<int4*>(&sh.id[l0]) = iv;
      }
    } else {
      for (int e = 0; e < 4 && i0 + e < nseg; ++e) {
        sh.key[l0 + e] = __float_as_uint(sc[base + i0 + e]);
        if (HAS_IDS) sh.id[l0 + e] = ids[base + i0 + e];
      }
    }
  }
  __syncthreads();
  const int i_own = tid * ITEMS;                 // first position of this thread's run
  uint32_t* krun = &sh.key[tid * RUN];
  const int32_t* irun = HAS_IDS ? &sh.id[tid * RUN] : nullptr;
  // reads of the own run, 4 items per 16-byte LDS access
  auto read_keys = [&](uint32_t (&k)[ITEMS]) {
#pragma unroll
    for (int q = 0; q < ITEMS / 4; ++q) {
      const uint4 v = *reinterpret_cast<const uint4*>(krun + 4 * q);
      k[4 * q] = v.x; k[4 * q + 1] = v.y; k[4 * q + 2] = v.z; k[4 * q + 3] = v.w;
    }
  };
  auto read_nids = [&](uint32_t (&nd)[ITEMS]) {
#pragma unroll
    for (int q = 0; q < ITEMS / 4; ++q) {
      if (HAS_IDS) {
        const int4 v = *reinterpret_cast<const int4*>(irun + 4 * q);
        nd[4 * q] = ~uint32_t(v.x); nd[4 * q + 1] = ~uint32_t(v.y);
        nd[4 * q + 2] = ~uint32_t(v.z); nd[4 * q + 3] = ~uint32_t(v.w);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) nd[4 * q + e] = ~uint32_t(base + i_own + 4 * q + e);
      }
    }
  };
  // 2. decode own run: validity, order keys (written back), key range
  uint32_t valid = 0;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  {
    uint32_t k[ITEMS], nd[ITEMS];
    read_keys(k);
    read_nids(nd);
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int32_t v = int32_t(~nd[i]);
      const bool ok = i_own + i < nseg && v >= 0 && v < lim;
      k[i] = ok ? order_key(__uint_as_float(k[i])) : 0u;
      if (ok) {
        valid |= 1u << i;
        kmin = k[i] < kmin ? k[i] : kmin;
        kmax = k[i] > kmax ? k[i] : kmax;
      }
    }
#pragma unroll
    for (int q = 0; q < ITEMS / 4; ++q)
      *reinterpret_cast<uint4*>(krun + 4 * q) =
          make_uint4(k[4 * q], k[4 * q + 1], k[4 * q + 2], k[4 * q + 3]);
  }
  const int lane = lane_id(), wave = tid >> 6;
  uint32_t nv = __popc(valid);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    nv += __shfl_xor(nv, o);
    const uint32_t x = __shfl_xor(kmin, o), y = __shfl_xor(kmax, o);
    kmin = x < kmin ? x : kmin;
    kmax = y > kmax ? y : kmax;
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

  uint32_t sel = valid;
  if (n > K) {
    const uint32_t range = kmax - kmin;
    const int bl = range ? 32 - __clz(range) : 0;
    int hi = bl ? 31 + bl : 31;   // highest bit any composite (key - kmin) << 32 | ~id can set
    uint32_t cm = valid;
    // sampled bound: histogram the first ITEMS/8 items of every run on the first digit, take
    // the bin whose upper tail should hold ~2K items; when that verifiably leaves between K
    // and kListCap candidates (the K-th largest is then among them), gather them (position
    // order) into the LDS list and finish on the list alone
    uint32_t list_n = 0;
    if (ITEMS >= 8) {
      constexpr int JS = ITEMS / 8;
      const int w0 = hi + 1 < 11 ? hi + 1 : 11;
      const int lo0 = hi + 1 - w0;
      const uint32_t msk0 = (1u << w0) - 1u;
      for (int b = tid; b < kBins; b += kTopkThreads) sh.hist[b] = 0;
      __syncthreads();
      uint32_t k[ITEMS], nd[ITEMS];
      read_keys(k);
      read_nids(nd);
      uint32_t ns = 0;
#pragma unroll
      for (int i = 0; i < JS; ++i)
        if ((valid >> i) & 1u) {
          atomicAdd(&sh.hist[digit_at(k[i] - kmin, nd[i], lo0, msk0)], 1u);
          ++ns;
        }
      ns = block_sum(ns, sh);
      uint32_t t = uint32_t((2ull * K * ns + n - 1) / n) + 16u;
      if (t > ns) t = ns;
      if (t > 0) {
        find_bin(sh, t);
        const uint32_t Ds = sh.s_digit;
        uint32_t c2 = 0;
#pragma unroll
        for (int i = 0; i < ITEMS; ++i)
          if (((valid >> i) & 1u) && digit_at(k[i] - kmin, nd[i], lo0, msk0) >= Ds) c2 |= 1u << i;
        uint32_t tot;
        uint32_t off = block_excl_scan(__popc(c2), sh, &tot);
        if (tot >= K && tot <= uint32_t(kListCap)) {
#pragma unroll
          for (int i = 0; i < ITEMS; ++i)
            if ((c2 >> i) & 1u) { sh.lkd[off] = k[i] - kmin; sh.lnid[off] = nd[i]; ++off; }
          list_n = tot;
          __syncthreads();
        } else if (tot >= K) {
          cm = c2;
        }
      }
    }
    if (list_n) {
      // ---- list path: thread t owns list items [t*L, (t+1)*L), L <= kListPerThread
      const int L = int((list_n + kTopkThreads - 1) / kTopkThreads);
      const int j0 = tid * L;
      int jn = int(list_n) - j0;
      jn = jn < 0 ? 0 : (jn > L ? L : jn);
      uint32_t lm = jn >= 32 ? 0xffffffffu : ((1u << jn) - 1u);
      Thresh T{hi + 1, 0, K, false};
      while (!T.done && hi >= 0) {
        const int w = hi + 1 < 11 ? hi + 1 : 11;
        const int lo = hi + 1 - w;
        const uint32_t msk = (1u << w) - 1u;
        for (int b = tid; b < kBins; b += kTopkThreads) sh.hist[b] = 0;
        __syncthreads();
        for (int q = 0; q < jn; ++q)
          if ((lm >> q) & 1u) atomicAdd(&sh.hist[digit_at(sh.lkd[j0 + q], sh.lnid[j0 + q], lo, msk)], 1u);
        __syncthreads();
        find_bin(sh, T.need);
        const uint32_t D = sh.s_digit;
        T.need -= sh.s_above;
        if (sh.hist[D] == T.need) T.done = true;
        T.P = (T.P << w) | D;
        T.lo = lo;
        for (int q = 0; q < jn; ++q)
          if (((lm >> q) & 1u) && digit_at(sh.lkd[j0 + q], sh.lnid[j0 + q], lo, msk) != D)
            lm &= ~(1u << q);
        hi = lo - 1;
        __syncthreads();
      }
      // select list items at or above the threshold, then compact them (list order is
      // position order); items are read into registers before any staging write
      uint32_t ls = 0, leq = 0;
      uint32_t rk[kListPerThread], rn[kListPerThread];
#pragma unroll
      for (int q = 0; q < kListPerThread; ++q) {
        rk[q] = 0; rn[q] = 0;
        if (q < jn) {
          rk[q] = sh.lkd[j0 + q];
          rn[q] = sh.lnid[j0 + q];
          const uint64_t v = prefix_at(rk[q], rn[q], T.lo);
          if (v > T.P) ls |= 1u << q;
          else if (v == T.P) leq |= 1u << q;
        }
      }
      if (T.done) {
        ls |= leq;
      } else {
        uint32_t tot;
        uint32_t before = block_excl_scan(__popc(leq), sh, &tot);
#pragma unroll
        for (int q = 0; q < kListPerThread; ++q)
          if ((leq >> q) & 1u) {
            if (before < T.need) ls |= 1u << q;
            ++before;
          }
      }
      uint32_t total;
      uint32_t o = block_excl_scan(__popc(ls), sh, &total);   // (barriers inside)
#pragma unroll
      for (int q = 0; q < kListPerThread; ++q)
        if ((ls >> q) & 1u) {
          sh.lnid[o] = rn[q];
          sh.lkd[o] = rk[q] + kmin;
          ++o;
        }
      __syncthreads();
      for (uint32_t kk = tid; kk < K; kk += kTopkThreads) {
        const bool has = kk < total;
        oi[kk] = has ? int32_t(~sh.lnid[kk]) : -1;
        if (os) os[kk] = has ? key_to_score(sh.lkd[kk]) : neg_inf();
      }
      __syncthreads();
      return;
    }
    // exact MSB-first radix over the candidates (every run)
    Thresh T{hi + 1, 0, K, false};
    while (!T.done && hi >= 0) {
      const int w = hi + 1 < 11 ? hi + 1 : 11;
      const int lo = hi + 1 - w;
      const uint32_t msk = (1u << w) - 1u;
      for (int b = tid; b < kBins; b += kTopkThreads) sh.hist[b] = 0;
      __syncthreads();
      uint32_t k[ITEMS], nd[ITEMS];
      read_keys(k);
      read_nids(nd);
#pragma unroll
      for (int i = 0; i < ITEMS; ++i)
        if ((cm >> i) & 1u) atomicAdd(&sh.hist[digit_at(k[i] - kmin, nd[i], lo, msk)], 1u);
      __syncthreads();
      find_bin(sh, T.need);
      const uint32_t D = sh.s_digit;
      T.need -= sh.s_above;
      if (sh.hist[D] == T.need) T.done = true;
      T.P = (T.P << w) | D;
      T.lo = lo;
#pragma unroll
      for (int i = 0; i < ITEMS; ++i)
        if (((cm >> i) & 1u) && digit_at(k[i] - kmin, nd[i], lo, msk) != D) cm &= ~(1u << i);
      hi = lo - 1;
      __syncthreads();
    }
    // final selection against the exact threshold
    sel = 0;
    uint32_t eq = 0;
    {
      uint32_t k[ITEMS], nd[ITEMS];
      read_keys(k);
      read_nids(nd);
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        if ((valid >> i) & 1u) {
          const uint64_t v = prefix_at(k[i] - kmin, nd[i], T.lo);
          if (v > T.P) sel |= 1u << i;
          else if (v == T.P) eq |= 1u << i;
        }
      }
    }
    if (T.done) {
      sel |= eq;
    } else {
      // duplicate ids left equal composites: keep the first T.need of them in position order
      uint32_t tot;
      uint32_t before = block_excl_scan(__popc(eq), sh, &tot);
#pragma unroll
      for (int i = 0; i < ITEMS; ++i)
        if ((eq >> i) & 1u) {
          if (before < T.need) sel |= 1u << i;
          ++before;
        }
    }
  }

  // ordered compaction (positions ascend with thread and item), staged in the list arrays
  uint32_t total;
  uint32_t o = block_excl_scan(__popc(sel), sh, &total);
  if (sel) {
    uint32_t k[ITEMS], nd[ITEMS];
    read_keys(k);
    read_nids(nd);
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
      if ((sel >> i) & 1u) {
        sh.lnid[o] = nd[i];
        sh.lkd[o] = k[i];
        ++o;
      }
  }
  __syncthreads();
  for (uint32_t k = tid; k < K; k += kTopkThreads) {
    const bool has = k < total;
    oi[k] = has ? int32_t(~sh.lnid[k]) : -1;
    if (os) os[k] = has ? key_to_score(sh.lkd[k]) : neg_inf();
  }
  __syncthreads();
}

template <int ITEMS, bool HAS_IDS>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkLevel L) {
  __shared__ Shared<HAS_IDS> sh;
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
}

template <int ITEMS, bool HAS_IDS>
hipError_t launch_level(const TopkLevel& L, int64_t rows, int64_t nseg, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(nseg), static_cast<unsigned>(rows));
  hipLaunchKernelGGL((topk_kernel<ITEMS, HAS_IDS>), grid, dim3(kTopkThreads), 0, s, L);
  return hipGetLastError();
}

hipError_t run_level(const TopkLevel& L, int64_t rows, int64_t nseg, hipStream_t s) {
  const int64_t seg = L.seg;
  if (L.ids) {
    if (seg <= 4 * kTopkThreads) return launch_level<4, true>(L, rows, nseg, s);
    if (seg <= 8 * kTopkThreads) return launch_level<8, true>(L, rows, nseg, s);
    return launch_level<16, true>(L, rows, nseg, s);
  }
  if (seg <= 4 * kTopkThreads) return launch_level<4, false>(L, rows, nseg, s);
  if (seg <= 8 * kTopkThreads) return launch_level<8, false>(L, rows, nseg, s);
  if (seg <= 16 * kTopkThreads) return launch_level<16, false>(L, rows, nseg, s);
  return launch_level<32, false>(L, rows, nseg, s);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return v ? atoi(v) : dflt;
}
// Tuning override (read once): positions per segment.
int64_t tune_seg() {
  static const int64_t v = [] {
    int64_t x = env_int("CSA_TUNE_TOPK_SEG", int(kSegMax));
    return x >= 2048 && x <= kSegMax ? (x + 2047) / 2048 * 2048 : kSegMax;
  }();
  return v;
}

// Scratch layout: two ping-pong candidate buffers (ids, scores) sized by the first level.
struct Plan {
  int64_t seg, nseg;
};
constexpr int64_t kSegIds = int64_t(kMaxItemsIds) * kTopkThreads;
Plan plan(int64_t n, bool has_ids) {
  Plan p{};
  p.seg = has_ids ? kSegIds : tune_seg();
  if (n <= p.seg) return p;
  p.nseg = ceil_div(n, p.seg);
  return p;
}

}  // namespace

size_t topk_scratch_bytes(int64_t rows, int64_t max_count, int K) {
  // the larger of the two plans (implicit / explicit ids)
  const Plan a = plan(max_count, false), b = plan(max_count, true);
  const int64_t ns = a.nseg > b.nseg ? a.nseg : b.nseg;
  return size_t(4) * rows * ns * K * 4;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  const int64_t n = a.max_count < 1 ? 1 : a.max_count;
  const Plan p = plan(n, a.ids != nullptr);
  if (p.nseg == 0) {
    TopkLevel L{a.scores, a.stride, a.ids, a.id_stride, a.id_limit, a.count, n, n, a.K,
                a.out_idx, a.out_score, a.out_stride};
    return run_level(L, a.rows, 1, s);
  }
  const int64_t per = a.rows * p.nseg * a.K;
  char* base = reinterpret_cast<char*>(a.scratch);
  int32_t* idb[2] = {reinterpret_cast<int32_t*>(base),
                     reinterpret_cast<int32_t*>(base + per * 4)};
  float* scb[2] = {reinterpret_cast<float*>(base + 2 * per * 4),
                   reinterpret_cast<float*>(base + 3 * per * 4)};
  // level 0: segments of the rows
  TopkLevel L0{a.scores, a.stride, a.ids, a.id_stride, a.id_limit, a.count, n, p.seg, a.K,
               idb[0], scb[0], p.nseg * a.K};
  hipError_t e = run_level(L0, a.rows, p.nseg, s);
  if (e != hipSuccess) return e;
  int cur = 0;
  int64_t m = p.nseg * a.K;   // candidates per row at the current level
  while (true) {
    if (m <= kSegIds) {
      TopkLevel Lf{scb[cur], m, idb[cur], m, nullptr, nullptr, m, m, a.K, a.out_idx,
                   a.out_score, a.out_stride};
      return run_level(Lf, a.rows, 1, s);
    }
    const int64_t ns = ceil_div(m, kSegIds);
    TopkLevel Lm{scb[cur], m, idb[cur], m, nullptr, nullptr, m, kSegIds, a.K, idb[cur ^ 1],
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
