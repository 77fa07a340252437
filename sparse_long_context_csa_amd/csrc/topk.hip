// Top-K selection, block maxima and the hierarchical candidate pool.
//
// "DeepSeek V4-Flash: The Cost of Deciding What to Read", section "The Lightning Indexer":
// a cheap scoring pass picks the top 512 entries and attention runs over those; section
// "FP4, down to the index scores": the selector decides on FP32 index scores.
// "DeepSeek-V4.1-Flash's KV-Cache Compression, Checked Down to the Byte", section 3, and the
// "DeepSeek-V4.1-Flash" study, "Hierarchical indexing bounds the deeper searches": blocks
// of 8 positions scored by their maximum, at most 2,048 blocks kept as a candidate pool.
//
// Selection rule (exact, integer): positions are ordered by the order-preserving key of their
// fp32 score, then by lower position (positions ascend with ids), and the chosen ids are
// written in ascending order, -1 padded.
//
// Threshold select.
//  * The bound: a lower bound T of a row's K-th largest score. The row is cut into G > K
//    disjoint groups of positions; the K-th largest group maximum is reached by at least K
//    distinct positions (each of those groups holds its own maximum), so it cannot exceed the
//    K-th largest score. The groups are built from the 16-position maxima that the scan
//    writes (long rows) or from the scores themselves, f at a time, so that G falls in
//    [2K, 8K) when the row is long enough; T then admits only a small fraction of positions
//    beyond K. T is that group maximum with the key bits below two 11-bit radix digits
//    cleared (digits taken from the top of the group maxima's key range).
//  * The candidates: the positions whose key reaches T, kept in position order.
//  * The select: an exact MSB-first radix select over LDS histograms of the candidates
//    (digits from the top of their key range); equal keys at the boundary are taken lowest
//    position first, and the chosen positions are compacted in order. When the candidates
//    exceed the LDS list, the same select streams over the row's scores instead: exact for
//    any input, slow only when tens of thousands of scores crowd above T.
// Rows of up to 32,768 positions take one workgroup each for all three steps
// (select_row_kernel). Longer rows whose scan left per-chunk candidate segments take one
// workgroup each over those segments (select_chunks_kernel, exactness checked against the
// chunks' own thresholds, see there). Other long rows are cut into slices of 4,096
// positions: one workgroup per slice computes the bound and keeps its slice's candidates in a
// segment of its own (select_slice_kernel), then one workgroup per row concatenates the
// segments in position order and selects (select_final_kernel).
#include <algorithm>
#include <type_traits>
#include <limits.h>
#include <stdlib.h>

#include "csa_common.hpp"
#include "ingest.hpp"
#include "launch.hpp"

namespace csa {

namespace {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kDigit0 = 14;            // bits of the final select's first digit
constexpr int kBins0 = 1 << kDigit0;
constexpr int kDigitB = 12;            // bits of the bound's digit
constexpr int kBinsB = 1 << kDigitB;   // (its histogram also serves the later digits)
constexpr int kDigit = 11;             // bits of the later digits
constexpr int kGroup = 32;             // bins per group count
constexpr int kSliceItems = 8;                        // positions per thread
constexpr int kSlice = kSelThreads * kSliceItems;     // positions per workgroup
constexpr int kSegCap = 512;           // candidates one slice workgroup keeps
constexpr int kListCap = 8192;         // candidates the final select holds in LDS
constexpr int kListRun = kListCap / kSelThreads;
constexpr int kMaxSegLds = 1024;       // segments whose offsets the final select keeps in LDS
constexpr int kSegPerThread = kMaxSegLds / kSelThreads;
constexpr int kCoarseCap = 16384;      // group maxima for the bound (< 8K, K <= 2048)
constexpr int64_t kRowMax = 32768;     // rows up to this length: one workgroup per row
constexpr int kHead = 32;              // segment entries loaded with the counts
constexpr int kHeadPerThread = 4;

struct SelArgs {
  const float* scores;
  int64_t stride;
  const uint32_t* gmax;   // 16-position maxima of the scores as order keys, or null
  int64_t gstride;
  const int32_t* ids;     // null: id = position
  int64_t id_stride;
  const int32_t* id_limit;
  const int32_t* count;
  int64_t max_count;
  uint32_t K;
  int32_t* out_idx;
  float* out_score;
  int64_t out_stride;
  uint2* bound;           // [rows] (T, largest key of the row)
  int32_t* seg_n;         // [rows][nseg] candidates found (may exceed kSegCap)
  uint2* seg;             // [rows][nseg][kSegCap] (key, position)
  int64_t nseg;
  int64_t rows;
  int64_t n_side;         // ingest workgroups after the rows' (0: none)
  int side_parts;         // ... 1 + side_parts per sequence with query preparation (else 1):
                          // part 0 runs the ingest, parts 1 .. side_parts prepare the queries
  IngestArgs side;
  SegArgs cseg;           // candidate segments of the decode scan (cseg.seg null: none)
  int key_floor;          // 16 when every score is a bf16 value: keys differing below bit 16
                          // of their offset from the list minimum are equal
};

// Side workgroup i of a decode step: sequence i % n_seq, part i / n_seq. Part 0 runs the
// sequence's ingest (without the indexer keys); parts 1 .. side_parts share the preparation of
// the attention calls' queries when the step asks for it (kept off part 0, whose ingest is the
// longest side job).
__device__ __forceinline__ void side_ingest(const SelArgs& a, int64_t i) {
  const int64_t sq = i % a.side.n_seq;
  const int part = int(i / a.side.n_seq);
  if (part == 0) {
    for (int v = threadIdx.x; v < ingest_vectors(a.side); v += blockDim.x) {
      if (a.side.dt == kBF16) ingest_vector<uint16_t>(a.side, sq, v, false);
      else ingest_vector<float>(a.side, sq, v, false);
    }
  }
  if (a.side.n_qprep > 0 && part > 0) {   // the attention calls' queries, off its path
    if (a.side.dt == kBF16) prep_queries<uint16_t>(a.side, sq, part - 1, a.side_parts);
    else prep_queries<float>(a.side, sq, part - 1, a.side_parts);
  }
}

struct SelShared {
  union {
    uint32_t coarse[kCoarseCap];                                    // the bound
    struct { uint32_t lk[kListCap]; uint32_t lp[kListCap]; } list;   // the select
  };
  uint32_t h0[kBins0];              // first digit of the select
  uint32_t h0g[kBins0 / kGroup];
  uint32_t hb[kBinsB];              // digit of the bound; later digits of the select
  uint32_t hbg[kBinsB / kGroup];
  uint32_t segoff[kMaxSegLds + 4];
  uint32_t wred[kSelWaves];
  uint32_t res[4];                  // search result: bin, items above it, items in it
  uint32_t red[4];                  // block reductions: min, max, count
  uint32_t flag;
};

__device__ __forceinline__ int64_t row_count(const SelArgs& a, int64_t r) {
  const int64_t n = a.count[r];
  return n < 0 ? 0 : (n > a.max_count ? a.max_count : n);
}

// the same through the scalar cache (r uniform; count[] is written by an earlier kernel, and a
// kernel starts with the scalar cache invalidated): the wait for it counts scalar loads only,
// so vector loads issued before its use are not waited for with it
__device__ __forceinline__ int64_t row_count_s(const SelArgs& a, int64_t r) {
  const int64_t n = *(const __attribute__((address_space(4))) int32_t*)(a.count + r);
  return n < 0 ? 0 : (n > a.max_count ? a.max_count : n);
}

__device__ __forceinline__ int64_t row_limit(const SelArgs& a, int64_t r) {
  return a.id_limit ? int64_t(a.id_limit[r]) : int64_t(INT_MAX);
}

__device__ __forceinline__ int key_bits(uint32_t range) { return range ? 32 - __clz(range) : 1; }

// exclusive prefix sum over the block; *total receives the block sum
__device__ __forceinline__ uint32_t excl_scan(uint32_t v, uint32_t* wred, uint32_t* total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t u = __shfl_up(x, o);
    if (lane >= o) x += u;
  }
  if (lane == kWave - 1) wred[wave] = x;
  __syncthreads();
  uint32_t add = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const uint32_t t = wred[w];
    if (w < wave) add += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return x - v + add;
}

__device__ __forceinline__ void clear_words(uint32_t* p, int n) {
  for (int b = threadIdx.x * 4; b < n; b += kSelThreads * 4)
    *reinterpret_cast<uint4*>(p + b) = make_uint4(0u, 0u, 0u, 0u);
}

__device__ __forceinline__ void hist_add(uint32_t* h, uint32_t* g, uint32_t bin) {
  atomicAdd(&h[bin], 1u);
  atomicAdd(&g[bin / kGroup], 1u);
}

// Search of a histogram of nbins = 2^w bins (and its 32-bin group counts) for the bin that
// holds the need-th largest item (1 <= need <= total). Wave 0 alone: each lane sums up to 8
// group counts from the top, a wave scan finds the group, a second one the bin. Results in
// sh.res after the barrier that ends the call.
__device__ __forceinline__ void wave_find(SelShared& sh, const uint32_t* h, const uint32_t* g,
                                          int nbins, uint32_t need) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int gsz = nbins < kGroup ? nbins : kGroup;
    const int ng = nbins / gsz;
    const int gpl = (ng + kWave - 1) / kWave;   // <= 8
    uint32_t c[8], sum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int gi = ng - 1 - lane * gpl - i;
      c[i] = (i < gpl && gi >= 0) ? g[gi] : 0u;
      sum += c[i];
    }
    uint32_t x = sum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t u = __shfl_up(x, o);
      if (lane >= o) x += u;
    }
    uint32_t acc = x - sum, gab = 0;
    int gsel = -1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (gsel < 0 && acc < need && need <= acc + c[i]) { gsel = ng - 1 - lane * gpl - i; gab = acc; }
      acc += c[i];
    }
    const uint64_t m = __ballot(gsel >= 0);
    const int src = m ? __ffsll(static_cast<unsigned long long>(m)) - 1 : 0;
    const int G = __shfl(gsel, src);
    const uint32_t GA = __shfl(gab, src);
    const int bin = (G < 0 ? 0 : G) * gsz + gsz - 1 - lane;
    const uint32_t hv = lane < gsz ? h[bin] : 0u;
    uint32_t y = hv;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t u = __shfl_up(y, o);
      if (lane >= o) y += u;
    }
    const uint32_t ex = GA + y - hv;
    if (lane < gsz && ex < need && need <= ex + hv) {
      sh.res[0] = uint32_t(bin); sh.res[1] = ex; sh.res[2] = hv;
    }
  }
  __syncthreads();
}

// The K-th key's bin (prefix P at shift lo, in_bin items of which `need` are to be taken)
// holds at most 64 items: rank them directly rather than by further digits. Each thread's
// items of the bin go to tmp (LDS, 64 words free for the call), wave 0 finds the need-th
// largest key X of the bin; returns (X - kmin, items of the bin above X, items equal to X)
// for the select to continue at full key resolution. Ends with a barrier.
template <int N>
__device__ __forceinline__ uint3 rank_bin(SelShared& sh, uint32_t* tmp, const uint32_t (&k)[N],
                                          uint32_t jn, uint32_t kmin, int lo, uint32_t P,
                                          uint32_t in_bin, uint32_t need) {
  const int tid = threadIdx.x;
  if (tid == 0) sh.flag = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (uint32_t(i) < jn && ((k[i] - kmin) >> lo) == P) tmp[atomicAdd(&sh.flag, 1u)] = k[i];
  __syncthreads();
  if (tid < kWave) {
    const uint32_t mine = uint32_t(tid) < in_bin ? tmp[tid] : 0u;
    uint32_t gt = 0, eq = 0;
    for (uint32_t j = 0; j < in_bin; ++j) {
      const uint32_t o = tmp[j];
      gt += o > mine;
      eq += o == mine;
    }
    // the key with gt < need <= gt + eq is the K-th; lanes holding it agree
    if (uint32_t(tid) < in_bin && gt < need && need <= gt + eq) {
      sh.res[0] = mine - kmin;
      sh.res[1] = gt;
      sh.res[2] = eq;
    }
  }
  __syncthreads();
  return make_uint3(sh.res[0], sh.res[1], sh.res[2]);
}

// Radix state: items with ((key - kmin) >> lo) > P are taken, those equal to P too when
// done, else the first `need` of them in position order.
struct Radix {
  uint32_t P;
  int lo;
  uint32_t need;
  bool done;
};

// state after a first-digit search (bin, above, count in sh.res) at shift lo
__device__ __forceinline__ Radix radix_first(const SelShared& sh, uint32_t K, int lo) {
  Radix st;
  st.P = sh.res[0];
  st.lo = lo;
  st.need = K - sh.res[1];
  st.done = sh.res[2] == st.need;
  return st;
}

// Further 11-bit digits over the items that `each(fn)` presents (fn(key) per item of this
// thread) until the bin of the K-th item is taken whole or all bits are resolved.
template <typename Each>
__device__ __forceinline__ void radix_more(SelShared& sh, Each each, uint32_t kmin, Radix& st) {
#pragma unroll 1
  while (!st.done && st.lo > 0) {
    const int w = st.lo < kDigit ? st.lo : kDigit;
    const int lw = st.lo, l = lw - w;
    const int nbins = 1 << w;
    clear_words(sh.hb, nbins < 4 ? 4 : nbins);
    if (threadIdx.x < kBinsB / kGroup) sh.hbg[threadIdx.x] = 0u;
    __syncthreads();
    const uint32_t P = st.P;
    each([&](uint32_t k) {
      const uint32_t v = k - kmin;
      if ((v >> lw) == P) hist_add(sh.hb, sh.hbg, (v >> l) & uint32_t(nbins - 1));
    });
    __syncthreads();
    wave_find(sh, sh.hb, sh.hbg, nbins, st.need);
    st.need -= sh.res[1];
    st.P = (st.P << w) | sh.res[0];
    st.lo = l;
    st.done = sh.res[2] == st.need;
    __syncthreads();
  }
}

__device__ __forceinline__ void write_out(const SelArgs& a, int64_t r, uint32_t o, uint32_t pos,
                                          uint32_t key) {
  a.out_idx[r * a.out_stride + o] = a.ids ? a.ids[r * a.id_stride + pos] : int32_t(pos);
  if (a.out_score) a.out_score[r * a.out_stride + o] = key_to_score(key);
}

__device__ __forceinline__ void pad_out(const SelArgs& a, int64_t r, uint32_t from) {
  for (uint32_t k = from + threadIdx.x; k < a.K; k += kSelThreads) {
    a.out_idx[r * a.out_stride + k] = -1;
    if (a.out_score) a.out_score[r * a.out_stride + k] = neg_inf();
  }
}

// The chosen items leave through LDS: each thread stages its items at their output slots
// (position and key in sh.h0, whose histogram is no longer needed), then one pass writes the
// K slots in order, each lane one consecutive slot (padding past nsel), so the global stores
// coalesce instead of following each thread's scattered slots.
constexpr int kMaxK = 2048;
static_assert(2 * kMaxK <= kBins0, "output staging lives in the first-digit histogram");
__device__ __forceinline__ void stage_out(SelShared& sh, uint32_t o, uint32_t pos, uint32_t key) {
  sh.h0[o] = pos;
  sh.h0[kMaxK + o] = key;
}
__device__ __forceinline__ void flush_out(const SelArgs& a, SelShared& sh, int64_t r,
                                          uint32_t nsel) {
  __syncthreads();
  for (uint32_t k = threadIdx.x; k < a.K; k += kSelThreads) {
    if (k < nsel) {
      const uint32_t pos = sh.h0[k];
      a.out_idx[r * a.out_stride + k] = a.ids ? a.ids[r * a.id_stride + pos] : int32_t(pos);
      if (a.out_score) a.out_score[r * a.out_stride + k] = key_to_score(sh.h0[kMaxK + k]);
    } else {
      a.out_idx[r * a.out_stride + k] = -1;
      if (a.out_score) a.out_score[r * a.out_stride + k] = neg_inf();
    }
  }
}

// block min / max / count through sh.red (initialised, and made visible, beforehand)
__device__ __forceinline__ void red_add(SelShared& sh, uint32_t kmin, uint32_t kmax, uint32_t c) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t x = __shfl_xor(kmax, o), y = __shfl_xor(kmin, o);
    kmax = x > kmax ? x : kmax;
    kmin = y < kmin ? y : kmin;
    c += __shfl_xor(c, o);
  }
  if (lane_id() == 0) {
    atomicMin(&sh.red[0], kmin);
    atomicMax(&sh.red[1], kmax);
    atomicAdd(&sh.red[2], c);
  }
}
__device__ __forceinline__ void red_init(SelShared& sh) {
  if (threadIdx.x == 0) { sh.red[0] = 0xffffffffu; sh.red[1] = 0u; sh.red[2] = 0u; }
}

// ---- the bound ---------------------------------------------------------------------------
// T and the row's largest key (all-ones when unknown). Needs sh.hb/hbg clear and sh.red
// initialised (and a barrier since); ends with a barrier.
__device__ __forceinline__ uint2 row_bound(const SelArgs& a, SelShared& sh, int64_t r, int64_t n) {
  const int tid = threadIdx.x;
  const int64_t K = a.K;
  if (n <= K) return make_uint2(0u, 0xffffffffu);
  const int64_t n16 = (n + 15) / 16;
  const bool use_g = a.gmax != nullptr && n16 >= 2 * K;
  const uint32_t* gsrc = use_g ? a.gmax + r * a.gstride : nullptr;   // keys
  const float* ssrc = a.scores + r * a.stride;                       // scores
  const int64_t nb = use_g ? n16 : n;
  int64_t f = nb / (4 * K);
  if (f < 1) f = 1;
  const int64_t G = (nb + f - 1) / f;   // K < G < 8K
  const uint32_t kninf = order_key(neg_inf());
  uint32_t kmax = 0u, kmin = 0xffffffffu, cf = 0;
  auto note = [&](int64_t j, uint32_t k) {
    sh.coarse[j] = k;
    if (k > kninf) {
      kmax = k > kmax ? k : kmax;
      kmin = k < kmin ? k : kmin;
      ++cf;
    }
  };
  // key of source element p (a 16-position maximum, or one score)
  auto key_at = [&](int64_t p) -> uint32_t { return use_g ? gsrc[p] : order_key(ssrc[p]); };
  if (f == 8) {
    // the long-row case: two 16-byte loads per group, 4 groups per thread in flight
    constexpr int kPer = 4;
    for (int64_t j0 = 0; j0 < G; j0 += int64_t(kPer) * kSelThreads) {
      uint4 v[kPer][2];
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int64_t j = j0 + tid + int64_t(q) * kSelThreads;
        const int64_t p0 = j * 8;
        v[q][0] = make_uint4(kninf, kninf, kninf, kninf);
        v[q][1] = v[q][0];
        if (j < G && p0 + 8 <= nb) {
          if (use_g) {
            v[q][0] = *reinterpret_cast<const uint4*>(gsrc + p0);
            v[q][1] = *reinterpret_cast<const uint4*>(gsrc + p0 + 4);
          } else {
            const float4 x0 = *reinterpret_cast<const float4*>(ssrc + p0);
            const float4 x1 = *reinterpret_cast<const float4*>(ssrc + p0 + 4);
            v[q][0] = make_uint4(order_key(x0.x), order_key(x0.y), order_key(x0.z), order_key(x0.w));
            v[q][1] = make_uint4(order_key(x1.x), order_key(x1.y), order_key(x1.z), order_key(x1.w));
          }
        } else if (j < G) {
          uint32_t* e8 = reinterpret_cast<uint32_t*>(&v[q][0]);
          uint32_t* e8b = reinterpret_cast<uint32_t*>(&v[q][1]);
          for (int e = 0; e < 8 && p0 + e < nb; ++e) (e < 4 ? e8[e] : e8b[e - 4]) = key_at(p0 + e);
        }
      }
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int64_t j = j0 + tid + int64_t(q) * kSelThreads;
        if (j < G) {
          const uint32_t m0 = max(max(v[q][0].x, v[q][0].y), max(v[q][0].z, v[q][0].w));
          const uint32_t m1 = max(max(v[q][1].x, v[q][1].y), max(v[q][1].z, v[q][1].w));
          note(j, max(m0, m1));
        }
      }
    }
  } else if (f == 4 && G <= 16 * kSelThreads && !use_g) {
    // four scores per group: group j is the float4 at 4 j (rows are 16-byte aligned); all of a
    // thread's groups (at most 16) load at once, coalesced across the lanes
    constexpr int kQ = 16;
    float4 v[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int64_t j = tid + int64_t(q) * kSelThreads;
      v[q] = j < G && 4 * j + 4 <= nb ? *reinterpret_cast<const float4*>(ssrc + 4 * j)
                                      : make_float4(neg_inf(), neg_inf(), neg_inf(), neg_inf());
    }
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int64_t j = tid + int64_t(q) * kSelThreads;
      if (j >= G) continue;
      uint32_t m;
      if (4 * j + 4 <= nb) {
        m = max(max(order_key(v[q].x), order_key(v[q].y)), max(order_key(v[q].z), order_key(v[q].w)));
      } else {   // the row's partial last group
        m = 0u;
        for (int64_t p = 4 * j; p < nb; ++p) m = max(m, order_key(ssrc[p]));
      }
      note(j, m);
    }
  } else if (f == 1 && G > 2 * kSelThreads && G <= 16 * kSelThreads) {
    // one element per group, more than two per thread (the prefill's rows of 32K positions,
    // 2,048 groups): all of a thread's elements (at most 4, 8 or 16, by G) load in one round,
    // none masked (indices past the last read the last one, unused), instead of one round
    // trip each (at two per thread, the loop below measured faster)
    auto one_round = [&](auto qn) {
      constexpr int kQ = decltype(qn)::value;
      uint32_t v[kQ];
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        const int64_t j = tid + int64_t(q) * kSelThreads;
        v[q] = key_at(j < G ? j : G - 1);
      }
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        const int64_t j = tid + int64_t(q) * kSelThreads;
        if (j < G) note(j, v[q]);
      }
    };
    if (G <= 4 * kSelThreads) one_round(std::integral_constant<int, 4>());
    else if (G <= 8 * kSelThreads) one_round(std::integral_constant<int, 8>());
    else one_round(std::integral_constant<int, 16>());
  } else {
    for (int64_t j = tid; j < G; j += kSelThreads) {
      const int64_t p0 = j * f;
      const int64_t p1 = p0 + f < nb ? p0 + f : nb;
      uint32_t m = 0u;
      for (int64_t p = p0; p < p1; ++p) {
        const uint32_t k = key_at(p);
        m = k > m ? k : m;
      }
      note(j, m);
    }
  }
  red_add(sh, kmin, kmax, cf);
  __syncthreads();
  kmin = sh.red[0];
  kmax = sh.red[1];
  cf = sh.red[2];
  // fewer than K finite groups: every valid position is a candidate
  if (cf < uint32_t(K)) return make_uint2(0u, kmax);
  // one 12-bit digit of (key - kmin): T within 2^(bits - 12) below the K-th group maximum
  const int bits = key_bits(kmax - kmin);
  const int w = bits < kDigitB ? bits : kDigitB;
  const int lo = bits - w;
  for (int64_t j = tid; j < G; j += kSelThreads) {
    const uint32_t k = sh.coarse[j];
    if (k > kninf) hist_add(sh.hb, sh.hbg, (k - kmin) >> lo);
  }
  __syncthreads();
  wave_find(sh, sh.hb, sh.hbg, 1 << w, uint32_t(K));
  return make_uint2(kmin + (sh.res[0] << lo), kmax);
}

// first-digit layout of the select over candidates with keys in [kmin, kmax]
struct Digit0 {
  int lo, nbins;
};
__device__ __forceinline__ Digit0 digit0(uint32_t kmin, uint32_t kmax) {
  const int bits = key_bits(kmax > kmin ? kmax - kmin : 0u);
  const int w = bits < kDigit0 ? bits : kDigit0;
  return Digit0{bits - w, 1 << w};
}
__device__ __forceinline__ uint32_t bin0(uint32_t k, uint32_t kmin, const Digit0& d0) {
  const uint32_t b = (k > kmin ? k - kmin : 0u) >> d0.lo;
  return b < uint32_t(d0.nbins) ? b : uint32_t(d0.nbins - 1);
}

// ---- the select --------------------------------------------------------------------------
// Candidates in LDS (position order), more than K of them, first digit (14 bits at lo0 over
// key - kmin) already histogrammed in sh.h0: thread t owns list items [t*L, t*L + L).
// `unsafe(T)` (per thread; any thread true rejects) is asked, once the radix has fixed the
// K-th key's prefix, whether the list may miss positions whose key reaches T = kmin + (that
// prefix << its shift), a lower bound of the K-th key. Then nothing is written and the call
// returns false with T in *t_lb.
struct NeverUnsafe {
  __device__ bool operator()(uint32_t) const { return false; }
};
template <typename Unsafe = NeverUnsafe>
__device__ __forceinline__ bool select_list(const SelArgs& a, SelShared& sh, int64_t r, uint32_t total,
                            uint32_t kmin, int lo0, int nb0, Unsafe unsafe = Unsafe(),
                            uint32_t* t_lb = nullptr, bool build_h0 = false) {
  const int tid = threadIdx.x;
  const uint32_t K = a.K;
  const uint32_t L = (total + kSelThreads - 1) / kSelThreads;   // <= kListRun
  const uint32_t j0 = uint32_t(tid) * L;
  const uint32_t jn = j0 < total ? (total - j0 < L ? total - j0 : L) : 0u;
  uint32_t k[kListRun];
#pragma unroll
  for (int i = 0; i < kListRun; ++i) k[i] = uint32_t(i) < jn ? sh.list.lk[j0 + i] : 0u;
  if (build_h0) {   // the first digit from this thread's run (sh.h0 / h0g clear beforehand)
#pragma unroll
    for (int i = 0; i < kListRun; ++i)
      if (uint32_t(i) < jn) hist_add(sh.h0, sh.h0g, bin0(k[i], kmin, Digit0{lo0, nb0}));
    __syncthreads();
  }
  wave_find(sh, sh.h0, sh.h0g, nb0, K);
  Radix st = radix_first(sh, K, lo0);
  const uint32_t in_bin = sh.res[2];
  __syncthreads();
  if (!st.done && st.lo > 0 && in_bin <= uint32_t(kWave)) {
    const uint3 x = rank_bin(sh, sh.hb, k, jn, kmin, st.lo, st.P, in_bin, st.need);
    st.P = x.x;
    st.need -= x.y;
    st.done = x.z == st.need;
    st.lo = 0;
  }
  radix_more(sh, [&](auto fn) {
#pragma unroll
    for (int i = 0; i < kListRun; ++i)
      if (uint32_t(i) < jn) fn(k[i]);
  }, kmin, st);
  if (t_lb) {
    const uint32_t T = kmin + (st.lo >= 32 ? 0u : (st.P << st.lo));
    if (tid == 0) sh.flag = 0u;
    __syncthreads();
    if (unsafe(T)) atomicOr(&sh.flag, 1u);
    __syncthreads();
    if (sh.flag) {
      *t_lb = T;
      return false;
    }
  }
  uint32_t sel = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < kListRun; ++i) {
    if (uint32_t(i) < jn) {
      const uint32_t v = (k[i] - kmin) >> st.lo;
      if (v > st.P) sel |= 1u << i;
      else if (v == st.P) eq |= 1u << i;
    }
  }
  if (st.done) {
    sel |= eq;
  } else {
    uint32_t tot;
    uint32_t before = excl_scan(__popc(eq), sh.wred, &tot);
#pragma unroll
    for (int i = 0; i < kListRun; ++i)
      if ((eq >> i) & 1u) {
        if (before < st.need) sel |= 1u << i;
        ++before;
      }
  }
  uint32_t nsel;
  uint32_t o = excl_scan(__popc(sel), sh.wred, &nsel);
#pragma unroll
  for (int i = 0; i < kListRun; ++i)
    if ((sel >> i) & 1u) {
      stage_out(sh, o, sh.list.lp[j0 + i], k[i]);
      ++o;
    }
  flush_out(a, sh, r, nsel);
  return true;
}

// the first `total` (<= K) list items, in order
__device__ __forceinline__ void select_all(const SelArgs& a, SelShared& sh, int64_t r, uint32_t total) {
  for (uint32_t j = threadIdx.x; j < total; j += kSelThreads)
    write_out(a, r, j, sh.list.lp[j], sh.list.lk[j]);
  pad_out(a, r, total);
}

// Streaming select over the row's scores (valid positions whose key reaches T): for rows
// whose candidates do not fit the LDS list. Uses every histogram; needs nothing set up.
__device__ __forceinline__ void select_stream(const SelArgs& a, SelShared& sh, int64_t r, int64_t n,
                              uint32_t T) {
  const int tid = threadIdx.x;
  const int64_t lim = row_limit(a, r);
  const float* sr = a.scores + r * a.stride;
  auto item = [&](int64_t p, uint32_t& k) -> bool {
    if (p >= n) return false;
    k = order_key(sr[p]);
    if (k < T) return false;
    const int64_t id = a.ids ? int64_t(a.ids[r * a.id_stride + p]) : p;
    return id >= 0 && id < lim;
  };
  __syncthreads();
  red_init(sh);
  clear_words(sh.h0, kBins0);
  clear_words(sh.h0g, kBins0 / kGroup);
  __syncthreads();
  uint32_t cnt = 0, kmin = 0xffffffffu, kmax = 0u;
  for (int64_t p = tid; p < n; p += kSelThreads) {
    uint32_t k;
    if (item(p, k)) {
      ++cnt;
      kmin = k < kmin ? k : kmin;
      kmax = k > kmax ? k : kmax;
    }
  }
  red_add(sh, kmin, kmax, cnt);
  __syncthreads();
  kmin = sh.red[0];
  kmax = sh.red[1];
  const uint32_t total = sh.red[2];
  Radix st{0u, 32, 0u, true};   // lo = 32: every candidate taken
  if (total > a.K) {
    const int bits = key_bits(kmax - kmin);
    const int w = bits < kDigit0 ? bits : kDigit0;
    const int lo0 = bits - w;
    for (int64_t p = tid; p < n; p += kSelThreads) {
      uint32_t k;
      if (item(p, k)) hist_add(sh.h0, sh.h0g, (k - kmin) >> lo0);
    }
    __syncthreads();
    wave_find(sh, sh.h0, sh.h0g, 1 << w, a.K);
    st = radix_first(sh, a.K, lo0);
    __syncthreads();
    radix_more(sh, [&](auto fn) {
      for (int64_t p = tid; p < n; p += kSelThreads) {
        uint32_t k;
        if (item(p, k)) fn(k);
      }
    }, kmin, st);
  }
  // ordered compaction, tile by tile
  uint32_t out_base = 0, eq_base = 0;
  for (int64_t t0 = 0; t0 < n; t0 += kSlice) {
    const int64_t q0 = t0 + int64_t(tid) * kSliceItems;
    uint32_t k[kSliceItems];
    uint32_t sel = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < kSliceItems; ++i) {
      k[i] = 0u;
      if (item(q0 + i, k[i])) {
        if (st.lo >= 32) {
          sel |= 1u << i;
        } else {
          const uint32_t v = (k[i] - kmin) >> st.lo;
          if (v > st.P) sel |= 1u << i;
          else if (v == st.P) eq |= 1u << i;
        }
      }
    }
    if (st.done) {
      sel |= eq;
    } else {
      uint32_t tot;
      uint32_t before = eq_base + excl_scan(__popc(eq), sh.wred, &tot);
#pragma unroll
      for (int i = 0; i < kSliceItems; ++i)
        if ((eq >> i) & 1u) {
          if (before < st.need) sel |= 1u << i;
          ++before;
        }
      eq_base += tot;
    }
    uint32_t tsel;
    uint32_t o = out_base + excl_scan(__popc(sel), sh.wred, &tsel);
#pragma unroll
    for (int i = 0; i < kSliceItems; ++i)
      if ((sel >> i) & 1u) {
        write_out(a, r, o, uint32_t(q0 + i), k[i]);
        ++o;
      }
    out_base += tsel;
  }
  pad_out(a, r, out_base);
}

// load N scores of positions q0.. (0 beyond n); N a multiple of 4
template <int N = kSliceItems>
__device__ __forceinline__ void load_slice(const float* sr, int64_t q0, int64_t n, float (&x)[N]) {
  if (q0 + N <= n) {
#pragma unroll
    for (int v = 0; v < N / 4; ++v) {
      const float4 y = *reinterpret_cast<const float4*>(sr + q0 + 4 * v);
      x[4 * v] = y.x; x[4 * v + 1] = y.y; x[4 * v + 2] = y.z; x[4 * v + 3] = y.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = q0 + i < n ? sr[q0 + i] : 0.f;
  }
}
// candidate flags (bit i: position q0 + i is a valid id whose key reaches T) and order keys
template <int N = kSliceItems>
__device__ __forceinline__ uint32_t slice_flags(const SelArgs& a, int64_t r, int64_t q0,
                                                int64_t n, int64_t lim, uint32_t T,
                                                const float (&x)[N], uint32_t (&key)[N]) {
  static_assert(N <= 32, "flags are 32 bits");
  // A candidate list's scan scores its invalid ids (-1, or past the row's visible count) -inf:
  // only a position whose score is -inf needs its id read back to tell the two apart.
  const uint32_t kninf = order_key(neg_inf());
  uint32_t flags = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int64_t p = q0 + i;
    key[i] = order_key(x[i]);
    bool ok = p < n && key[i] >= T;
    if (ok && key[i] <= kninf) {
      const int64_t id = a.ids ? int64_t(a.ids[r * a.id_stride + p]) : p;
      ok = id >= 0 && id < lim;
    }
    if (ok) flags |= 1u << i;
  }
  return flags;
}

// Rows up to kRowMax: one workgroup per row. Thread t holds the kRun consecutive positions
// [b + t kRun, + kRun) of each block of kRowBlock positions (the first block is loaded before
// the bound is computed, so its loads overlap that); the candidates (keys at or above the
// bound T, in position order) go to the LDS list with one prefix scan per block.
constexpr int kRun = 32;
constexpr int64_t kRowBlock = int64_t(kRun) * kSelThreads;
// x: this thread's run of the row's first block, loaded (positions past n are not read)
__device__ __forceinline__ void select_row_rest(const SelArgs& a, SelShared& sh, int64_t r,
                                                int64_t n, float (&x)[kRun]) {
  const int tid = threadIdx.x;
  const float* sr = a.scores + r * a.stride;
  clear_words(sh.h0, kBins0);
  clear_words(sh.h0g, kBins0 / kGroup);
  clear_words(sh.hb, kBinsB);
  clear_words(sh.hbg, kBinsB / kGroup);
  red_init(sh);
  __syncthreads();
  const uint2 B = row_bound(a, sh, r, n);
  const uint32_t T = B.x;
  const Digit0 d0 = digit0(T, B.y);
  const int64_t lim = row_limit(a, r);
  uint32_t total = 0;
  bool over = false;
  for (int64_t b = 0; b < n; b += kRowBlock) {
    const int64_t q0 = b + int64_t(tid) * kRun;
    uint32_t key[kRun];
    const uint32_t flags = slice_flags<kRun>(a, r, q0, n, lim, T, x, key);
    if (b + kRowBlock < n) load_slice<kRun>(sr, q0 + kRowBlock, n, x);
    uint32_t tot;
    uint32_t off = total + excl_scan(__popc(flags), sh.wred, &tot);
    if (total + tot <= uint32_t(kListCap)) {
#pragma unroll
      for (int i = 0; i < kRun; ++i)
        if ((flags >> i) & 1u) {
          sh.list.lk[off] = key[i];
          sh.list.lp[off] = uint32_t(q0 + i);
          ++off;
        }
    } else {
      over = true;
    }
    total += tot;
  }
  __syncthreads();
  if (over) select_stream(a, sh, r, n, T);
  else if (total <= a.K) select_all(a, sh, r, total);
  else select_list(a, sh, r, total, T, d0.lo, d0.nbins, NeverUnsafe(), nullptr, true);
}

__device__ __forceinline__ void select_row_body(const SelArgs& a, SelShared& sh, int64_t r,
                                                int64_t n) {
  float x[kRun];
  load_slice<kRun>(a.scores + r * a.stride, int64_t(threadIdx.x) * kRun, n, x);
  select_row_rest(a, sh, r, n, x);
}

__global__ __launch_bounds__(kSelThreads) void select_row_kernel(SelArgs a) {
  __shared__ SelShared sh;
  if (int64_t(blockIdx.x) >= a.rows) {
    side_ingest(a, int64_t(blockIdx.x) - a.rows);
    return;
  }
  const int64_t r = blockIdx.x;
  // The first block's scores load before the row's count is known, up to the buffer's
  // capacity (max_count; positions at or past the count are read but never used), so that
  // the count's round trip and theirs overlap; the empty asm keeps them ahead of it.
  float x[kRun];
  load_slice<kRun>(a.scores + r * a.stride, int64_t(threadIdx.x) * kRun, a.max_count, x);
  asm volatile("" ::: "memory");
  select_row_rest(a, sh, r, row_count_s(a, r), x);
}

// Rows whose decode scan left candidate segments (SegArgs): one workgroup per row. Chunk c
// holds every position of the chunk whose key reaches its tau_c, so the segments
// concatenated in chunk order form a list in position order; thread t holds the run
// [t*L, t*L + L) of it in registers. An MSB-first radix select with 11-bit digits over a
// 2,048-bin LDS histogram finds the K-th key of the list; the chosen positions leave in
// list order (ascending), equal keys at the boundary lowest position first.
// The result is the row's exact Top-K when every tau_c is at or below the K-th key of the
// list: a position missing from the list then lies below that key, hence outside the row's
// Top-K as well. The check uses the lower bound kmin + (prefix << shift) of the K-th key that
// the radix has fixed. A chunk that fails it sends the row to the streaming select with that
// bound; an overflowing segment or a list longer than the registers hold, with bound 0.
// Short rows of the batch (<= kRowMax) take the single-row select.
constexpr int kSegDigit = 11;
constexpr int kSegBins = 1 << kSegDigit;
constexpr int kSegRun = 16;                          // list items per thread
constexpr int kSegList = kSelThreads * kSegRun;      // 8,192
constexpr int kSegHead = 32;                         // entries fetched with the counts
constexpr int kSegHeadIters = 8;                     // rounds of 32 chunks fetched that way
constexpr int kSegHeadChunks = kSegHeadIters * (kSelThreads / 16);

// bin (of nbins, counted from the top by thread order: thread t owns the 4 bins
// [nbins - 4t - 4, nbins - 4t)) that holds the need-th largest item; writes (bin, items above
// it, items in it) to sh.res. All threads; ends with a barrier.
__device__ __forceinline__ void seg_find(SelShared& sh, const uint32_t* h, int nbins,
                                         uint32_t need) {
  const int tid = threadIdx.x;
  const int b0 = nbins - 4 * tid - 1;                // this thread's highest bin
  uint32_t c[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[i] = b0 - i >= 0 ? h[b0 - i] : 0u;
    sum += c[i];
  }
  uint32_t tot;
  uint32_t acc = excl_scan(sum, sh.wred, &tot);
  if (acc < need && need <= acc + sum) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (acc < need && need <= acc + c[i]) {
        sh.res[0] = uint32_t(b0 - i); sh.res[1] = acc; sh.res[2] = c[i];
      }
      acc += c[i];
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kSelThreads) void select_chunks_kernel(SelArgs a) {
  __shared__ SelShared sh;
  if (int64_t(blockIdx.x) >= a.rows) {
    side_ingest(a, int64_t(blockIdx.x) - a.rows);
    return;
  }
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const SegArgs& sg = a.cseg;
  // 1. one round of independent loads, issued before the row's count is known rather than
  //    after it: the counts and thresholds of every chunk the buffers hold (2 per thread) and the
  //    first kSegHead entries of the first kSegHeadChunks chunks (16 lanes per chunk, 2 entries
  //    per lane). Chunks past the row's visible ones are read (in bounds, stale) and ignored.
  const int64_t ncap = sg.nseg < kMaxSegLds ? sg.nseg : kMaxSegLds;
  const int lane16 = tid & 15;
  // (indices past the buffers' chunks read their last one: no load is masked, so all of them
  // go out back to back)
  uint4 hv[kSegHeadIters];
#pragma unroll
  for (int it = 0; it < kSegHeadIters; ++it) {
    int64_t ch = int64_t(it) * (kSelThreads / 16) + (tid >> 4);
    ch = ch < ncap ? ch : ncap - 1;
    hv[it] = *reinterpret_cast<const uint4*>(sg.seg + (r * sg.nseg + ch) * kChunkSegCap +
                                             2 * lane16);
  }
  uint32_t cn_l[kSegPerThread];
  uint2 info_l[kSegPerThread];
#pragma unroll
  for (int q = 0; q < kSegPerThread; ++q) {
    int64_t j = int64_t(tid) * kSegPerThread + q;
    j = j < ncap ? j : ncap - 1;
    cn_l[q] = uint32_t(sg.seg_n[r * sg.nseg + j]);
    info_l[q] = sg.seg_info[r * sg.nseg + j];
  }
  // keeps these loads here, ahead of the row's count and the branches on it (the compiler
  // would otherwise sink them into the long-row path, after the count's round trip); the
  // count's own wait then finds them in flight
  asm volatile("" ::: "memory");
  const int64_t n = row_count_s(a, r);
  if (n <= kRowMax) {
    select_row_body(a, sh, r, n);
    return;
  }
  const int64_t nch = (n + sg.chunk - 1) / sg.chunk;
  if (nch > kMaxSegLds) {
    select_stream(a, sh, r, n, 0u);
    return;
  }
  const uint32_t K = a.K;
  const uint32_t kninf = order_key(neg_inf());
  uint32_t c[kSegPerThread], tau[kSegPerThread], loc = 0;
  uint32_t tmin = 0xffffffffu, tmax = 0u;
  bool over = false;
#pragma unroll
  for (int q = 0; q < kSegPerThread; ++q) {
    const int64_t j = int64_t(tid) * kSegPerThread + q;
    c[q] = 0u;
    tau[q] = 0u;
    if (j < nch) {
      const uint32_t cn = cn_l[q];
      const uint2 info = info_l[q];
      over |= cn > uint32_t(kChunkSegCap);
      c[q] = cn < uint32_t(kChunkSegCap) ? cn : uint32_t(kChunkSegCap);
      tau[q] = info.x;
      tmin = info.x < tmin ? info.x : tmin;
      tmax = info.y > tmax ? info.y : tmax;
      loc += c[q];
    }
  }
  for (int b = tid; b < kSegBins; b += kSelThreads) sh.hb[b] = 0u;
  red_init(sh);
  if (tid == 0) {
    sh.flag = 0u;
    sh.red[3] = 0u;   // the largest chunk threshold
  }
  __syncthreads();
  bool rest = false;   // a chunk with entries past the fetched heads
#pragma unroll
  for (int q = 0; q < kSegPerThread; ++q) {
    const int64_t j = int64_t(tid) * kSegPerThread + q;
    if (j < nch && (c[q] > uint32_t(kSegHead) || j >= kSegHeadChunks)) rest = true;
  }
  if (over) atomicOr(&sh.flag, 1u);
  if (rest) atomicOr(&sh.flag, 2u);
  {
    uint32_t tq = 0u;
#pragma unroll
    for (int q = 0; q < kSegPerThread; ++q) tq = tau[q] > tq ? tau[q] : tq;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint32_t y = __shfl_xor(tq, o);
      tq = y > tq ? y : tq;
    }
    if ((tid & 63) == 0) atomicMax(&sh.red[3], tq);
  }
  red_add(sh, tmin, tmax, 0u);
  uint32_t total;
  uint32_t off = excl_scan(loc, sh.wred, &total);
#pragma unroll
  for (int q = 0; q < kSegPerThread; ++q) {
    const int64_t j = int64_t(tid) * kSegPerThread + q;
    if (j < nch) sh.segoff[j] = off;
    off += c[q];
  }
  if (tid == 0) sh.segoff[nch] = total;
  __syncthreads();
  // list keys are finite (above kninf) and reach their chunk's tau
  const uint32_t kmin = sh.red[0] > kninf ? sh.red[0] : kninf + 1u;
  const uint32_t kmax = sh.red[1] > kmin ? sh.red[1] : kmin;
  const uint32_t tau_max = sh.red[3];
  const uint32_t flag = sh.flag;
  if ((flag & 1u) != 0u || total > uint32_t(kSegList)) {
    select_stream(a, sh, r, n, 0u);
    return;
  }
  // 2. the list in LDS, in position order: the fetched heads, then (rarely) the rest
#pragma unroll
  for (int it = 0; it < kSegHeadIters; ++it) {
    const int64_t ch = int64_t(it) * (kSelThreads / 16) + (tid >> 4);
    if (ch < nch) {
      const uint32_t o0 = sh.segoff[ch], cn = sh.segoff[ch + 1] - o0;
      const uint32_t e = 2u * uint32_t(lane16);
      if (e < cn) { sh.list.lk[o0 + e] = hv[it].x; sh.list.lp[o0 + e] = hv[it].y; }
      if (e + 1 < cn) { sh.list.lk[o0 + e + 1] = hv[it].z; sh.list.lp[o0 + e + 1] = hv[it].w; }
    }
  }
  if (flag & 2u) {
    // entries past the heads: one wave per chunk
    const int wv = tid >> 6, ln = tid & 63;
    for (int64_t ch = wv; ch < nch; ch += kSelWaves) {
      const uint32_t o0 = sh.segoff[ch], cn = sh.segoff[ch + 1] - o0;
      const uint32_t e0 = ch < kSegHeadChunks ? uint32_t(kSegHead) : 0u;
      for (uint32_t e = e0 + ln; e < cn; e += 64) {
        const uint2 v = sg.seg[(r * sg.nseg + ch) * kChunkSegCap + e];
        sh.list.lk[o0 + e] = v.x;
        sh.list.lp[o0 + e] = v.y;
      }
    }
  }
  __syncthreads();
  // this thread's run of the list into registers; first-digit histogram
  const uint32_t L = (total + kSelThreads - 1) / kSelThreads;
  const uint32_t j0 = uint32_t(tid) * L;
  const uint32_t jn = j0 < total ? (total - j0 < L ? total - j0 : L) : 0u;
  const int bits = key_bits(kmax - kmin);
  int lo = bits > kSegDigit ? bits - kSegDigit : 0;
  uint32_t k[kSegRun], pos[kSegRun];
#pragma unroll
  for (int i = 0; i < kSegRun; ++i) {
    k[i] = 0u;
    pos[i] = 0u;
    if (uint32_t(i) < jn) {
      k[i] = sh.list.lk[j0 + i];
      pos[i] = sh.list.lp[j0 + i];
      atomicAdd(&sh.hb[(k[i] - kmin) >> lo], 1u);
    }
  }
  __syncthreads();
  if (total <= K) {
    // the list is the row's Top-K only if every chunk kept all its valid positions
    if (tau_max > kninf + 1u) {   // uniform
      select_stream(a, sh, r, n, 0u);
      return;
    }
#pragma unroll
    for (int i = 0; i < kSegRun; ++i)
      if (uint32_t(i) < jn) write_out(a, r, j0 + i, pos[i], k[i]);
    pad_out(a, r, total);
    return;
  }
  // 3. radix select: P = prefix of the K-th key at shift lo, need = items of it to take
  seg_find(sh, sh.hb, 1 << (bits - lo), K);
  uint32_t P = sh.res[0], need = K - sh.res[1];
  const uint32_t in_bin = sh.res[2];
  bool done = in_bin == need;
  if (!done && lo > 0 && in_bin <= uint32_t(kWave)) {
    const uint3 x = rank_bin(sh, sh.h0, k, jn, kmin, lo, P, in_bin, need);   // sh.h0 is free
    P = x.x;
    need -= x.y;
    done = x.z == need;
    lo = 0;
  }
  // with bf16-valued scores two different keys differ by at least 2^16 (their low 16 bits
  // depend only on the sign, and -0 reads as +0), so the bin at shift key_floor holds one key
#pragma unroll 1
  while (!done && lo > a.key_floor) {
    const int w = lo - a.key_floor < kSegDigit ? lo - a.key_floor : kSegDigit;
    const int l2 = lo - w;
    __syncthreads();
    for (int b = tid; b < (1 << w); b += kSelThreads) sh.hb[b] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSegRun; ++i) {
      const uint32_t v = k[i] - kmin;
      if (uint32_t(i) < jn && (v >> lo) == P) atomicAdd(&sh.hb[(v >> l2) & ((1u << w) - 1u)], 1u);
    }
    __syncthreads();
    seg_find(sh, sh.hb, 1 << w, need);
    P = (P << w) | sh.res[0];
    need -= sh.res[1];
    done = sh.res[2] == need;
    lo = l2;
  }
  // 4. exactness: every chunk's tau at or below the K-th key's lower bound
  const uint32_t T = kmin + (P << lo);
  if (tau_max > T) {   // uniform
    select_stream(a, sh, r, n, T);
    return;
  }
  // 5. chosen items in list order
  uint32_t sel = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < kSegRun; ++i)
    if (uint32_t(i) < jn) {
      const uint32_t v = (k[i] - kmin) >> lo;
      if (v > P) sel |= 1u << i;
      else if (v == P) eq |= 1u << i;
    }
  if (done) {
    sel |= eq;
  } else {
    uint32_t tot;
    uint32_t before = excl_scan(__popc(eq), sh.wred, &tot);
#pragma unroll
    for (int i = 0; i < kSegRun; ++i)
      if ((eq >> i) & 1u) {
        if (before < need) sel |= 1u << i;
        ++before;
      }
  }
  uint32_t nsel;
  uint32_t o = excl_scan(__popc(sel), sh.wred, &nsel);
#pragma unroll
  for (int i = 0; i < kSegRun; ++i)
    if ((sel >> i) & 1u) {
      stage_out(sh, o, pos[i], k[i]);
      ++o;
    }
  flush_out(a, sh, r, nsel);
}

// Long rows, step 1: one workgroup per slice computes the row's bound and keeps its slice's
// candidates (position order) in its segment; workgroup 0 of the row records the bound.
__global__ __launch_bounds__(kSelThreads) void select_slice_kernel(SelArgs a) {
  __shared__ SelShared sh;
  const int64_t r = blockIdx.y, b = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t n = row_count(a, r);
  const int64_t p0 = b * kSlice;
  if (p0 >= n) {
    if (tid == 0) {
      a.seg_n[r * a.nseg + b] = 0;
      if (b == 0) a.bound[r] = make_uint2(0u, 0xffffffffu);
    }
    return;
  }
  const int64_t q0 = p0 + int64_t(tid) * kSliceItems;
  const float* sr = a.scores + r * a.stride;
  float x[kSliceItems];
  load_slice(sr, q0, n, x);
  clear_words(sh.hb, kBinsB);
  clear_words(sh.hbg, kBinsB / kGroup);
  red_init(sh);
  __syncthreads();
  const uint2 B = row_bound(a, sh, r, n);
  uint32_t key[kSliceItems];
  const uint32_t flags = slice_flags(a, r, q0, n, row_limit(a, r), B.x, x, key);
  uint32_t tot;
  uint32_t off = excl_scan(__popc(flags), sh.wred, &tot);
  uint2* seg = a.seg + (r * a.nseg + b) * kSegCap;
#pragma unroll
  for (int i = 0; i < kSliceItems; ++i)
    if ((flags >> i) & 1u) {
      if (off < uint32_t(kSegCap)) seg[off] = make_uint2(key[i], uint32_t(q0 + i));
      ++off;
    }
  if (tid == 0) {
    a.seg_n[r * a.nseg + b] = int32_t(tot);
    if (b == 0) a.bound[r] = B;
  }
}

// Long rows, step 2: one workgroup per row gathers the segments in position order (their
// first kHead entries load together with the counts; the first digit is histogrammed on the
// way) and selects; overflowing rows stream.
__global__ __launch_bounds__(kSelThreads) void select_final_kernel(SelArgs a) {
  __shared__ SelShared sh;
  if (int64_t(blockIdx.x) >= a.rows) {
    side_ingest(a, int64_t(blockIdx.x) - a.rows);
    return;
  }
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t n = row_count(a, r);
  const int64_t ns = (n + kSlice - 1) / kSlice;
  const uint2 B = a.bound[r];
  if (ns <= kMaxSegLds) {
    const bool spec = ns * kHead <= int64_t(kSelThreads) * kHeadPerThread;
    uint2 hv[kHeadPerThread];
    if (spec) {
#pragma unroll
      for (int q = 0; q < kHeadPerThread; ++q) {
        const int idx = tid + q * kSelThreads;
        const int64_t sb = idx / kHead;
        hv[q] = sb < ns ? a.seg[(r * a.nseg + sb) * kSegCap + idx % kHead] : make_uint2(0u, 0u);
      }
    }
    uint32_t c[kSegPerThread], loc = 0;
    bool over = false, longseg = false;
#pragma unroll
    for (int q = 0; q < kSegPerThread; ++q) {
      const int64_t j = int64_t(tid) * kSegPerThread + q;
      c[q] = j < ns ? uint32_t(a.seg_n[r * a.nseg + j]) : 0u;
      over |= c[q] > uint32_t(kSegCap);
      longseg |= c[q] > uint32_t(kHead);
      loc += c[q];
    }
    clear_words(sh.h0, kBins0);
    clear_words(sh.h0g, kBins0 / kGroup);
    if (tid == 0) sh.flag = 0u;
    __syncthreads();
    if (over) atomicOr(&sh.flag, 1u);
    if (longseg) atomicOr(&sh.flag, 2u);
    uint32_t total;
    uint32_t off = excl_scan(loc, sh.wred, &total);
#pragma unroll
    for (int q = 0; q < kSegPerThread; ++q) {
      const int64_t j = int64_t(tid) * kSegPerThread + q;
      if (j < ns) sh.segoff[j] = off;
      off += c[q];
    }
    __syncthreads();
    const uint32_t flag = sh.flag;
    if ((flag & 1u) == 0u && total <= uint32_t(kListCap)) {
      const uint32_t T = B.x;
      const Digit0 d0 = digit0(T, B.y);
      const bool hist = total > a.K;
      if (spec) {
#pragma unroll
        for (int q = 0; q < kHeadPerThread; ++q) {
          const int idx = tid + q * kSelThreads;
          const int64_t sb = idx / kHead;
          if (sb < ns) {
            const uint32_t o0 = sh.segoff[sb];
            const uint32_t cb = (sb + 1 < ns ? sh.segoff[sb + 1] : total) - o0;
            const uint32_t e = uint32_t(idx % kHead);
            if (e < cb) {
              sh.list.lk[o0 + e] = hv[q].x;
              sh.list.lp[o0 + e] = hv[q].y;
              if (hist) hist_add(sh.h0, sh.h0g, bin0(hv[q].x, T, d0));
            }
          }
        }
      }
      if (!spec || (flag & 2u)) {
        // list slot j comes from the last segment whose offset is <= j
        for (uint32_t j = tid; j < total; j += kSelThreads) {
          int lo = 0, hi = int(ns) - 1;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sh.segoff[mid] <= j) lo = mid;
            else hi = mid - 1;
          }
          const uint32_t e = j - sh.segoff[lo];
          if (spec && e < uint32_t(kHead)) continue;
          const uint2 v = a.seg[(r * a.nseg + lo) * kSegCap + e];
          sh.list.lk[j] = v.x;
          sh.list.lp[j] = v.y;
          if (hist) hist_add(sh.h0, sh.h0g, bin0(v.x, T, d0));
        }
      }
      __syncthreads();
      if (!hist) select_all(a, sh, r, total);
      else select_list(a, sh, r, total, T, d0.lo, d0.nbins);
      return;
    }
  }
  select_stream(a, sh, r, n, B.x);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t round256(size_t x) { return (x + 255) / 256 * 256; }

struct SelPlan {
  bool split;
  int64_t nseg;
  size_t off_seg_n, off_seg, bytes;
};
SelPlan sel_plan(int64_t rows, int64_t max_count) {
  SelPlan p{};
  p.split = max_count > kRowMax;
  p.nseg = p.split ? ceil_div(max_count, kSlice) : 0;
  p.off_seg_n = round256(size_t(rows) * 8);
  p.off_seg = p.off_seg_n + round256(size_t(rows) * p.nseg * 4);
  p.bytes = p.off_seg + size_t(rows) * p.nseg * kSegCap * 8;
  return p;
}

}  // namespace

size_t topk_scratch_bytes(int64_t rows, int64_t max_count, int K) {
  (void)K;
  return sel_plan(rows, max_count).bytes;
}

hipError_t launch_topk(const TopkArgs& t, hipStream_t s) {
  if (t.rows == 0) return hipSuccess;
  const int64_t mc = t.max_count > 0 ? t.max_count : 0;
  const SelPlan p = sel_plan(t.rows, mc);
  char* base = reinterpret_cast<char*>(t.scratch);
  SelArgs a{};
  a.scores = t.scores; a.stride = t.stride; a.gmax = t.gmax; a.gstride = t.gstride;
  a.ids = t.ids; a.id_stride = t.id_stride; a.id_limit = t.id_limit; a.count = t.count;
  a.max_count = mc; a.K = uint32_t(t.K); a.out_idx = t.out_idx; a.out_score = t.out_score;
  a.out_stride = t.out_stride;
  a.bound = reinterpret_cast<uint2*>(base);
  a.seg_n = reinterpret_cast<int32_t*>(base + p.off_seg_n);
  a.seg = reinterpret_cast<uint2*>(base + p.off_seg);
  a.nseg = p.nseg;
  a.rows = t.rows;
  // query preparation: about two vectors per wave, so that no sequence's share waits on one
  // workgroup's bandwidth
  a.side_parts = 1;
  if (t.side && t.side->n_qprep > 0) {
    const int per_wg = 2 * (kSelThreads / 64);
    const int jobs = t.side->n_qprep * t.side->q_heads;
    a.side_parts = std::min(32, std::max(1, (jobs + per_wg - 1) / per_wg));
  }
  a.n_side = t.side ? t.side->n_seq * (1 + (t.side->n_qprep > 0 ? a.side_parts : 0)) : 0;
  a.side = t.side ? *t.side : IngestArgs{};
  a.cseg = t.seg;
  a.key_floor = t.bf16_scores ? 16 : 0;
  // with segments the scan leaves no 16-position maxima: short rows bound from the scores
  if (t.seg.seg != nullptr) a.gmax = nullptr;
  const unsigned rows = static_cast<unsigned>(t.rows);
  const unsigned last = static_cast<unsigned>(t.rows + a.n_side);   // + ingest workgroups
  if (t.seg.seg != nullptr) {
    hipLaunchKernelGGL(select_chunks_kernel, dim3(last), dim3(kSelThreads), 0, s, a);
    return hipGetLastError();
  }
  if (!p.split) {
    hipLaunchKernelGGL(select_row_kernel, dim3(last), dim3(kSelThreads), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(select_slice_kernel, dim3(static_cast<unsigned>(p.nseg), rows),
                     dim3(kSelThreads), 0, s, a);
  hipLaunchKernelGGL(select_final_kernel, dim3(last), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
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
