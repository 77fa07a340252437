// Lightning-indexer scan for many query rows (a prefill chunk): the one dense contraction of
// the path, on bf16 MFMA.
//
// "DeepSeek V4-Flash: The Cost of Deciding What to Read", section "The Lightning Indexer":
// I(t,s) = sum_h w(t,h) * ReLU(q_I(t,h) . k_I(s)); section "The indexer is O(n), and that is
// the ceiling": every visible entry is scored. Visibility: entry i is usable by a query at t
// only if m*(i+1)-1 <= t ("The sliding window is not an optimisation").
#include "csa_common.hpp"
#include "index_common.hpp"
#include "launch.hpp"

namespace csa {

namespace {

// ---- kPQ query rows per workgroup, 256-key tiles staged through LDS ------------------------
// One wave per query row (its 64 heads x 128 as the A operand in VGPRs); the workgroup's key
// tiles are shared by its rows. The next tile moves HBM -> LDS by LDS-DMA (issued from inline
// asm, no staging registers) while the current one is scored; one barrier per tile. Within a
// tile the MFMAs of 16-key group u+1 are issued (into the other accumulator set) before the
// ReLU, gate and head sum of group u, so the matrix pipe works while the VALU reduces, and the
// head sums of four groups are finished together with three row swaps.
constexpr int kPT = 256;          // keys per tile
static_assert(kPT % 64 == 0, "the score epilogue works on 4 groups of 16 keys at a time");

// Tile layout in LDS: blocks of 4 keys, 1,088 bytes apart; byte 16 l of block b holds the
// 16-byte chunk l >> 2 of key 4 b + (l & 3) (the layout of one LDS-DMA instruction).
constexpr int kPTBlocks = kPT / 4;
constexpr int kPTileBytes = kPTBlocks * kBlk;

__device__ __forceinline__ void read_group_Bd(const unsigned char* tile, int u, int g, int col,
                                              bf16x8_t (&B)[4]) {
  const unsigned char* rp = tile + (4 * u + (col >> 2)) * kBlk + (col & 3) * 16 + g * 64;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) B[ks] = *reinterpret_cast<const bf16x8_t*>(rp + ks * 256);
}

// LDS-DMA of block b of a tile (1 KiB: keys key0 .. key0 + 3). Issued from inline asm: the
// compiler's wait insertion, which cannot tell which LDS bytes a pending LDS-DMA writes, would
// otherwise make every read of the other tile buffer wait for this load. The issuing wave
// waits for its loads itself (vmcnt(0)) before the barrier that publishes the tile.
__device__ __forceinline__ void dma_block(const uint16_t* kb, int64_t key, unsigned char* dst,
                                          int lane) {
  const uint16_t* src = kb + key * kID + (lane >> 2) * 8;
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(
      uint32_t(size_t((const __attribute__((address_space(3))) unsigned char*)dst)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(src), "s"(m0v)
               : "memory", "m0");
}

template <int kPQ>
__global__ __launch_bounds__(kPQ * 64) void scan_prefill_kernel(ScanArgs a, int keys_per_block) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][kPTileBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
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

  const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.keys) + sq * a.e_cap * kID;
  // wave w moves blocks w, w + kPQ, ... of a tile (rows past k1 read the block's last row and
  // are not scored)
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto tload = [&](int64_t base, unsigned char* tile) {
    for (int b = wave_u; b < kPTBlocks; b += kPQ) {
      int64_t key = base + 4 * b + (lane & 3);
      key = key < k1 ? key : k1 - 1;
      dma_block(kb, key, tile + b * kBlk, lane);
    }
  };
  bf16x8_t A[4][4];
  load_query_A(reinterpret_cast<const uint16_t*>(a.q) + r * kIH * kID, lane, A);
  float wv[4][4];
  load_gates(a.w + r * kIH, lane, wv);
  tload(k0, lds[0]);
  float* out = a.scores + r * a.score_stride;
  uint32_t* gmax = a.gmax + r * a.gmax_stride;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  int buf = 0;
  for (int64_t base = k0; base < k1; base += kPT) {
    const bool more = base + kPT < k1;
    if (more) tload(base + kPT, lds[buf ^ 1]);
    if (base < n_vis) {
      const unsigned char* tile = lds[buf];
      const int nv = int(n_vis - base < kPT ? n_vis - base : kPT);   // visible in this tile
      float* ob = out + base;
      uint32_t* gb = gmax + (base >> 4);
      bf16x8_t B[4];
      f32x4_t acc[2][4];
      float scb[4];
      read_group_Bd(tile, 0, g, col, B);
      tile_mfma(A, B, acc[0]);
      const int grp = (g & 1) * 2 + (g >> 1);   // rows 0,1,2,3 hold groups 0,2,1,3
#pragma unroll
      for (int u = 0; u < kPT / 16; ++u) {
        if (u + 1 < kPT / 16) {
          read_group_Bd(tile, u + 1, g, col, B);
          tile_mfma(A, B, acc[(u + 1) & 1]);
        }
        scb[u & 3] = lane_part(acc[u & 1], wv);
        if (u + 1 < kPT / 16) {
          // issue order: the next group's 4 B reads, then each of its 16 MFMAs followed by
          // two VALU instructions of this group's epilogue
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
          }
        }
        if ((u & 3) == 3) {
          const float sv = sum_groups4(scb[0], scb[1], scb[2], scb[3]);
          const int p = (u - 3) * 16 + 16 * grp + col;
          if ((u - 3) * 16 + 64 <= nv) {
            ob[p] = sv;
            const uint32_t gk = max16_key(order_key_nz(sv));
            if (col == 0) gb[u - 3 + grp] = gk;
          } else if ((u - 3) * 16 < nv) {
            if (p < nv) ob[p] = sv;
            const uint32_t gk = max16_key(p < nv ? order_key_nz(sv) : order_key(neg_inf()));
            if (col == 0 && (u - 3 + grp) * 16 < nv) gb[u - 3 + grp] = gk;
          }
        }
      }
    }
    if (more) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      buf ^= 1;
    }
  }
}

}  // namespace

hipError_t launch_scan_prefill(const ScanArgs& a, int pq, int keys_per_block, dim3 grid,
                               hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (pq == 8)
    launch_k(scan_prefill_kernel<8>, grid, dim3(8 * 64), 0, s, e0, e1, a, keys_per_block);
  else
    launch_k(scan_prefill_kernel<12>, grid, dim3(12 * 64), 0, s, e0, e1, a, keys_per_block);
  return hipGetLastError();
}

}  // namespace csa
