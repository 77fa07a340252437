// MFMA core of the sparse attention (bf16, 64 heads x 512): one workgroup of 4 waves (16
// heads each) over one split of a query row's list of cached rows.
//
// "DeepSeek V4-Flash: The Cost of Deciding What to Read": sections "Key and value are the
// same vector", "Attention sink, and heads that abstain" and "The sliding window is not an
// optimisation" (the selected entries and the window rows form one softmax with the sink).
//
// The split's rows are walked in tiles of 32; each tile is gathered once into LDS twice:
// row-major (A operand of S^T = KV.Q^T, v_mfma_f32_16x16x32_bf16, M = 32 rows, N = 16 heads,
// K = 512) and transposed (B operand of O = P.V, K = 32 rows). The score accumulator layout
// puts, in every lane, 8 rows of one head; those 8 rows are exactly the lane's K slots of the
// P.V product, so P passes from the score registers to the A operand with no data movement.
// Online softmax in base 2. With one split the output is normalised (with the sink) and
// stored; with several, the split's (max, sum, unnormalised output) go to the workspace for
// attn_combine_kernel. row_src(j, nrows) gives the address of list row j (null: no row),
// which may point to global memory or LDS.
#pragma once

#include "csa_common.hpp"
#include "launch.hpp"

namespace csa {

constexpr int kAH = 64;          // heads on the MFMA path
constexpr int kAD = 512;         // head dim on the MFMA path
constexpr int kTile = 32;        // rows per tile
constexpr int kKvRow = 1040;     // LDS bytes per row of the row-major tile (1024 + 16)
constexpr int kVtRow = 80;       // LDS bytes per dim of the transposed tile (64 + 16)
constexpr float kLazyMax = 8.f;  // log2 headroom of the running softmax maximum

// Partials of split s of row r: the unnormalised output in the MFMA accumulator layout,
// [wave][nt][lane] 4 x bf16 (64 heads x 512 dims; each lane's 4 heads of one dim in 8 bytes),
// then, after every split's outputs, (max, sum) per head in base 2 as fp32 pairs. The output
// is rounded once to bf16 here; the maxima and sums stay fp32.
constexpr int64_t kPartO = int64_t(kAH) * kAD;   // elements per (row, split)

// two fp32 values rounded to bf16 (nearest even) by one v_cvt_pk_bf16_f32, low half first
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  bf16x2v_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint2 pack_bf16x4(const f32x4_t& v) {
  return make_uint2(cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3]));
}
// the 8-byte output cell (wave, nt, lane) of partial rs, and the (max, sum) pairs of rs
__device__ __forceinline__ uint2* part_out(void* ws, int64_t rs) {
  return reinterpret_cast<uint2*>(ws) + rs * (kPartO / 4);
}
__device__ __forceinline__ float2* part_ml(void* ws, int64_t n_parts, int64_t rs) {
  return reinterpret_cast<float2*>(reinterpret_cast<unsigned char*>(ws) + n_parts * kPartO * 2) +
         rs * kAH;
}


struct AttnLds {
  __attribute__((aligned(16))) unsigned char kvs[kTile * kKvRow];
  __attribute__((aligned(16))) unsigned char vts[kAD * kVtRow];
  int rowok[kTile];
};

template <class RowFn>
__device__ __forceinline__ void attn_split_mfma(const AttnArgs& a, AttnLds& L, int64_t r,
                                                int split, int nsplit, int tiles_per_split,
                                                int64_t n_rows_total, RowFn row_src) {
  unsigned char* kvs = L.kvs;
  unsigned char* vts = L.vts;
  int* rowok = L.rowok;
  const int nrows = a.top_k + a.window;
  const int64_t j0 = int64_t(split) * tiles_per_split * kTile;
  int64_t j1 = j0 + int64_t(tiles_per_split) * kTile;
  if (j1 > nrows) j1 = nrows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int head = 16 * wave + col;   // head of this lane in the score layout

  // gather assignment: thread -> rows 4*ra .. 4*ra+3 (ra = tid & 7), 16-byte chunks cp and
  // cp + 32 (cp = tid >> 3); rows past the list read the query row and are zeroed
  const int ra = tid & 7, cp = tid >> 3;
  const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + r * kAH * kAD;
  bf16x8_t vv[4][2];
  bool okr[4], f8r[4];
  const uint16_t* srcs[4];
  auto locate = [&](int64_t j) {   // row pointers of tile j (the ids load here)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      srcs[i] = row_src(j + 4 * ra + i, int(j1));
      okr[i] = srcs[i] != nullptr;
      f8r[i] = okr[i] && a.kv_fmt != kKvPlain && j + 4 * ra + i < a.top_k;
    }
  };
  // chunk c (dims 8c .. 8c+7) of a quantised entry. FP8: eight E4M3 codes at byte 8c (c < 56),
  // else eight bf16 values at byte 448 + 16 (c - 56); FP4: fp4_entry_chunk8
  auto chunk8 = [&](const uint16_t* row, int c) -> bf16x8_t {
    const uint8_t* e = reinterpret_cast<const uint8_t*>(row);
    if (a.kv_fmt == kKvFp4) return fp4_entry_chunk8(e, c);
    if (c < kFp8Nope / 8) {
      const uint2 w = *reinterpret_cast<const uint2*>(e + 8 * c);
      return e4m3x8_to_bf16(w.x, w.y);
    }
    return *reinterpret_cast<const bf16x8_t*>(e + kFp8Nope + 16 * (c - kFp8Nope / 8));
  };
  auto gather = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (f8r[i]) {
        vv[i][0] = chunk8(srcs[i], cp);
        vv[i][1] = chunk8(srcs[i], cp + 32);
        continue;
      }
      const uint16_t* sc = okr[i] ? srcs[i] : qrow;
      vv[i][0] = *reinterpret_cast<const bf16x8_t*>(sc + cp * 8);
      vv[i][1] = *reinterpret_cast<const bf16x8_t*>(sc + (cp + 32) * 8);
    }
  };
  if (j0 < j1) locate(j0);
  // Q^T as B operand: head `head`, dims ks*32 + g*8 .. +8 (loads while the ids arrive)
  bf16x8_t Qf[16];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + (r * kAH + head) * kAD + g * 8;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) Qf[ks] = *reinterpret_cast<const bf16x8_t*>(qp + ks * 32);
  }
  if (j0 < j1) gather();
  const float sl2 = a.scale * kLog2e;
  float m_run = neg_inf(), l_run = 0.f;
  f32x4_t O[32];
#pragma unroll
  for (int nt = 0; nt < 32; ++nt) O[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int64_t j = j0; j < j1; j += kTile) {
    // tile j to LDS: row-major (A operand of S^T) and transposed, 4 rows per 8-byte store
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!okr[i]) { vv[i][0] = bf16x8_t{}; vv[i][1] = bf16x8_t{}; }
      if (cp == 0) rowok[4 * ra + i] = okr[i];
      *reinterpret_cast<bf16x8_t*>(&kvs[(4 * ra + i) * kKvRow + cp * 16]) = vv[i][0];
      *reinterpret_cast<bf16x8_t*>(&kvs[(4 * ra + i) * kKvRow + (cp + 32) * 16]) = vv[i][1];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = cp + 32 * h;
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vv[0][h]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vv[1][h]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vv[2][h]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vv[3][h]);
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        // dims 2*e2 (low halves) and 2*e2+1 (high halves) of the 4 rows
        const uint32_t lo01 = __builtin_amdgcn_perm(w1[e2], w0[e2], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(w3[e2], w2[e2], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(w1[e2], w0[e2], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(w3[e2], w2[e2], 0x07060302u);
        *reinterpret_cast<uint2*>(&vts[(c * 8 + 2 * e2) * kVtRow + ra * 8]) = make_uint2(lo01, lo23);
        *reinterpret_cast<uint2*>(&vts[(c * 8 + 2 * e2 + 1) * kVtRow + ra * 8]) = make_uint2(hi01, hi23);
      }
    }
    __syncthreads();
    // the next tile's rows load while this one computes
    if (j + kTile < j1) {
      locate(j + kTile);
      gather();
    }

    // S^T: rows (4g+i) and (16+4g+i) against head `head`
    // four independent accumulator chains (even / odd K steps of both 16-row halves)
    f32x4_t S0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, S1 = S0, S2 = S0, S3 = S0;
#pragma unroll
    for (int ks = 0; ks < 16; ks += 2) {
      const bf16x8_t A0 = *reinterpret_cast<const bf16x8_t*>(&kvs[col * kKvRow + ks * 64 + g * 16]);
      const bf16x8_t A1 = *reinterpret_cast<const bf16x8_t*>(&kvs[(16 + col) * kKvRow + ks * 64 + g * 16]);
      const bf16x8_t A2 = *reinterpret_cast<const bf16x8_t*>(&kvs[col * kKvRow + ks * 64 + 64 + g * 16]);
      const bf16x8_t A3 = *reinterpret_cast<const bf16x8_t*>(&kvs[(16 + col) * kKvRow + ks * 64 + 64 + g * 16]);
      S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, Qf[ks], S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, Qf[ks], S1, 0, 0, 0);
      S2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A2, Qf[ks + 1], S2, 0, 0, 0);
      S3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A3, Qf[ks + 1], S3, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) { S0[i] += S2[i]; S1[i] += S3[i]; }
    float s[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = rowok[4 * g + i] ? S0[i] * sl2 : neg_inf();
      s[4 + i] = rowok[16 + 4 * g + i] ? S1[i] * sl2 : neg_inf();
    }
    float tmax = s[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, s[i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == neg_inf()) ? 1.f : exp2f(m_run - m_new);
    float p[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = (s[i] == neg_inf()) ? 0.f : exp2f(s[i] - m_new);
      psum += p[i];
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // P as the A operand: row = head `col`, K slots (g, i) <-> rows {4g..4g+3, 16+4g..16+4g+3}
    bf16x8_t Pf;
#pragma unroll
    for (int i = 0; i < 8; ++i) Pf[i] = (__bf16)p[i];
    // output rows are heads 4g+i of this wave: fetch their rescale factors
    float ai[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) O[nt][i] *= ai[i];
      const unsigned char* vp = &vts[(nt * 16 + col) * kVtRow];
      const uint2 lo = *reinterpret_cast<const uint2*>(vp + 8 * g);
      const uint2 hi = *reinterpret_cast<const uint2*>(vp + 32 + 8 * g);
      bf16x8_t Vf;
      const uint4 vv4 = make_uint4(lo.x, lo.y, hi.x, hi.y);
      Vf = *reinterpret_cast<const bf16x8_t*>(&vv4);
      O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Pf, Vf, O[nt], 0, 0, 0);
    }
    __syncthreads();
  }

  if (nsplit == 1) {
    const float zs = a.sink ? a.sink[head] * kLog2e : neg_inf();
    const float M = fmaxf(m_run, zs);
    float f = 0.f;
    if (M != neg_inf()) {
      const float em = (m_run == neg_inf()) ? 0.f : exp2f(m_run - M);
      const float den = l_run * em + ((zs == neg_inf()) ? 0.f : exp2f(zs - M));
      f = den > 0.f ? em / den : 0.f;
    }
    float fi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fi[i] = __shfl(f, 4 * g + i);
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + (r * kAH + 16 * wave) * kAD;
    const int rope0 = a.out_rope_dim > 0 ? kAD - a.out_rope_dim : kAD;
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) {
      float cs = 1.f, sn = 0.f;
      if (nt * 16 >= rope0)
        rope_cos_sin(-double(a.q_pos[r]), (nt * 16 + col - rope0) >> 1, a.out_rope_dim,
                     a.rope_log2_base, cs, sn);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float y = O[nt][i] * fi[i];
        if (nt * 16 >= rope0) y = rope_pair_lane(y, (col & 1) != 0, cs, sn);
        op[(4 * g + i) * kAD + nt * 16 + col] = f32_to_bf16(y);
      }
    }
  } else {
    // partial in the accumulator layout (8-byte stores), then (max, sum) per head
    const int64_t rs = r * nsplit + split;
    uint2* pp = part_out(a.ws, rs) + wave * 32 * kWave + lane;
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) pp[nt * kWave] = pack_bf16x4(O[nt]);
    if (g == 0) part_ml(a.ws, n_rows_total * nsplit, rs)[head] = make_float2(m_run, l_run);
  }
}


// ---- LDS-DMA tiles and transpose loads ----------------------------------------------------
// The same computation over tiles that arrive by LDS-DMA: each wave moves 8 of the tile's 32
// rows, one global_load_lds_dwordx4 per row (the row's 1 KiB lands contiguously, 1,040
// bytes apart), into one of two tile buffers while the other is computed. The list's row
// addresses are resolved once into LDS. S = KV.Q^T reads the row-major tile as before; the
// P.V operand (32 rows of one dim per lane) comes from the same row-major tile through the
// gfx950 transpose load ds_read_b64_tr_b16: within a 16-lane group, lane i supplies the
// address of row r0 + (i >> 2), dims d0 + 4 (i & 3), and lane j receives rows r0 .. r0 + 3
// of dim d0 + j. No transposed copy is built.
// Rows are 1,056 bytes apart (8 banks of shift per row), and the 16-byte chunk c of row r sits
// at chunk c ^ swz(r), swz(r) = (r >> 2) & 1, chosen by each DMA lane through its source
// address. The 16 lanes of a transpose load (rows 4k .. 4k+3, 32 bytes each) then cover the
// 32 banks once, and so do the 8 lanes of a score-operand read (rows r .. r+7, one chunk:
// rows 4 apart share a bank shift and differ in the swizzle).
constexpr int kMaxRowsLds = 1024;   // list rows of one split whose addresses fit in LDS
constexpr int kKvRowD = 1056;       // LDS bytes per row of a DMA tile

__device__ __forceinline__ int kv_swz(int row) { return (row >> 2) & 1; }

struct AttnDmaLds {
  __attribute__((aligned(16))) unsigned char kv[2][kTile * kKvRowD];
  const uint16_t* rowp[kMaxRowsLds];
  int rowok[2][kTile];
};

// one LDS-DMA row: 64 lanes x 16 bytes from src (per lane) to dst (uniform). From inline asm:
// the compiler's own wait insertion cannot tell which LDS bytes a pending LDS-DMA writes and
// would hold every read of the other tile buffer until it lands. The caller waits for its
// loads (vmcnt(0)) before the barrier that publishes the tile.
__device__ __forceinline__ void dma_row(const uint16_t* src, unsigned char* dst) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(
      uint32_t(size_t((const __attribute__((address_space(3))) unsigned char*)dst)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(m0v)
               : "memory", "m0");
}

typedef short v4s_t __attribute__((ext_vector_type(4)));

template <class RowFn>
__device__ __forceinline__ void attn_split_dma(const AttnArgs& a, AttnDmaLds& L, int64_t r,
                                               int split, int nsplit, int tiles_per_split,
                                               int64_t n_rows_total, RowFn row_src) {
  const int nrows = a.top_k + a.window;
  const int64_t j0 = int64_t(split) * tiles_per_split * kTile;
  int64_t j1 = j0 + int64_t(tiles_per_split) * kTile;
  if (j1 > nrows) j1 = nrows;
  const int nl = j1 > j0 ? int(j1 - j0) : 0;   // list rows of this split
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int g = lane >> 4, col = lane & 15;
  const int head = 16 * wave + col;   // head of this lane in the score layout
  const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + r * kAH * kAD;

  for (int i = tid; i < nl; i += blockDim.x) L.rowp[i] = row_src(j0 + i, int(j1));
  // Q^T as B operand: head `head`, dims ks*32 + g*8 .. +8
  bf16x8_t Qf[16];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + (r * kAH + head) * kAD + g * 8;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) Qf[ks] = *reinterpret_cast<const bf16x8_t*>(qp + ks * 32);
  }
  __syncthreads();
  // rows 8 w .. 8 w + 7 of tile t into buffer b; rows past the list (and rows without a
  // valid address) read the query row and are masked
  // A quantised entry row (kv_fmt FP8 or FP4, list row < top_k) moves as its raw bytes (576 or
  // 288: lanes 0 .. 35 or 0 .. 17 of the DMA; the others fetch query bytes into the rest of the
  // slot) and is expanded in place to the bf16 layout once it has landed (expand), which
  // rewrites all 1,024 bytes of the slot. qmask bit 8 b + i: row 8 w + i of buffer b.
  const int kvf = a.kv_fmt;
  const int raw_lanes = kvf == kKvFp8 ? kFp8EntryBytes / 16 : kFp4EntryBytes / 16;
  uint32_t qmask = 0u;
  auto issue = [&](int t, int b) {
    qmask &= ~(0xffu << (8 * b));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tr = 8 * wave_u + i;
      const int jr = t * kTile + tr;
      const uint16_t* p = jr < nl ? L.rowp[jr] : nullptr;
      const bool qz = p != nullptr && kvf != kKvPlain && j0 + jr < a.top_k;   // uniform
      if (qz) {
        const unsigned char* src = lane < raw_lanes
                                       ? reinterpret_cast<const unsigned char*>(p) + 16 * lane
                                       : reinterpret_cast<const unsigned char*>(qrow) + 16 * lane;
        dma_row(reinterpret_cast<const uint16_t*>(src), &L.kv[b][tr * kKvRowD]);
        qmask |= 1u << (8 * b + i);
      } else {
        dma_row((p != nullptr ? p : qrow) + (lane ^ kv_swz(tr)) * 8, &L.kv[b][tr * kKvRowD]);
      }
      if (lane == 0) L.rowok[b][tr] = p != nullptr;
    }
  };
  // this wave's quantised rows of buffer b, after their DMA has landed (vmcnt(0)): every lane
  // reads its raw bytes of each row before any lane writes (the writes use the reads' results
  // and each row is read by the same instructions), so the expansion may overwrite the raw bytes
  // in place; bf16 chunk c goes to slot chunk c ^ swz(row).
  // FP8: raw chunk l < 28 holds dims 16 l .. 16 l + 15 (bf16 chunks 2 l, 2 l + 1), raw chunk
  // 28 .. 35 the bf16 dims 448 + 8 (l - 28) .. (bf16 chunk l + 28).
  // FP4: lane (i, l) = (lane >> 4, lane & 15) expands code chunk l (dims 32 l .. 32 l + 31, bf16
  // chunks 4 l .. 4 l + 3) of rows h + i, h = 0 and 4, under the scales of blocks 2 l, 2 l + 1
  // (the two bytes at 256 + 2 l).
  auto expand8 = [&](int b, uint32_t bits) {
    // four rows' raw chunks are read together (one wait per four rows), then converted and
    // written
#pragma unroll
    for (int h = 0; h < 8; h += 4) {
      if (((bits >> h) & 0xfu) == 0u) continue;   // uniform
      uint4 raw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        raw[i] = make_uint4(0u, 0u, 0u, 0u);
        if (((bits >> (h + i)) & 1u) && lane < kFp8EntryBytes / 16)
          raw[i] = *reinterpret_cast<const uint4*>(
              &L.kv[b][(8 * wave_u + h + i) * kKvRowD + 16 * lane]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!((bits >> (h + i)) & 1u)) continue;   // uniform
        const int tr = 8 * wave_u + h + i;
        unsigned char* row = &L.kv[b][tr * kKvRowD];
        const int sw = kv_swz(tr);
        if (lane < kFp8Nope / 16) {
          const bf16x8_t lo = e4m3x8_to_bf16(raw[i].x, raw[i].y);
          const bf16x8_t hi = e4m3x8_to_bf16(raw[i].z, raw[i].w);
          *reinterpret_cast<bf16x8_t*>(row + 16 * ((2 * lane) ^ sw)) = lo;
          *reinterpret_cast<bf16x8_t*>(row + 16 * ((2 * lane + 1) ^ sw)) = hi;
        } else if (lane < kFp8EntryBytes / 16) {
          *reinterpret_cast<uint4*>(row + 16 * ((lane + kFp8Nope / 16) ^ sw)) = raw[i];
        }
      }
    }
  };
  auto expand4 = [&](int b, uint32_t bits) {
    const int qi = lane >> 4, ql = lane & 15;
    uint4 raw[2];
    uint32_t sc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      raw[h] = make_uint4(0u, 0u, 0u, 0u);
      sc[h] = 0u;
      if ((bits >> (4 * h + qi)) & 1u) {
        const unsigned char* row = &L.kv[b][(8 * wave_u + 4 * h + qi) * kKvRowD];
        raw[h] = *reinterpret_cast<const uint4*>(row + 16 * ql);
        sc[h] = *reinterpret_cast<const uint16_t*>(row + kFp4CodeBytes + 2 * ql);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (!((bits >> (4 * h + qi)) & 1u)) continue;
      const int tr = 8 * wave_u + 4 * h + qi;
      unsigned char* row = &L.kv[b][tr * kKvRowD];
      const int sw = kv_swz(tr);
      float s0, s1;
      e4m3x2_scales(sc[h], s0, s1);
      const bf16x8_t c0 = fp4x8_to_bf16(raw[h].x, s0);
      const bf16x8_t c1 = fp4x8_to_bf16(raw[h].y, s0);
      const bf16x8_t c2 = fp4x8_to_bf16(raw[h].z, s1);
      const bf16x8_t c3 = fp4x8_to_bf16(raw[h].w, s1);
      *reinterpret_cast<bf16x8_t*>(row + 16 * ((4 * ql) ^ sw)) = c0;
      *reinterpret_cast<bf16x8_t*>(row + 16 * ((4 * ql + 1) ^ sw)) = c1;
      *reinterpret_cast<bf16x8_t*>(row + 16 * ((4 * ql + 2) ^ sw)) = c2;
      *reinterpret_cast<bf16x8_t*>(row + 16 * ((4 * ql + 3) ^ sw)) = c3;
    }
  };
  auto expand = [&](int b) {
    const uint32_t bits = (qmask >> (8 * b)) & 0xffu;
    if (bits == 0u) return;   // uniform
    if (kvf == kKvFp4) expand4(b, bits);
    else expand8(b, bits);
  };
  const int ntiles = (nl + kTile - 1) / kTile;
  // Two tiles or fewer (the decode splits): both go out at once and land before the first
  // is computed, so the tile loop runs with no further wait, expansion or barrier.
  const bool all_in = ntiles <= 2;
  if (ntiles > 0) issue(0, 0);
  if (all_in && ntiles > 1) issue(1, 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // The query loads have landed with that wait, but the compiler does not see the LDS-DMA
  // loads or the wait (both asm): left alone, it would guard the tile loop's first use of Qf
  // with its own vmcnt(0), which also waits for the next tile's rows and so serialises the
  // double buffering. Using Qf here (an empty asm) retires them in its count once, at no cost.
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) asm volatile("" ::"v"(Qf[ks]));
  expand(0);
  if (all_in && ntiles > 1) expand(1);
  __syncthreads();

  const float sl2 = a.scale * kLog2e;
  float m_run = neg_inf(), l_run = 0.f;
  f32x4_t O[32];
#pragma unroll
  for (int nt = 0; nt < 32; ++nt) O[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < ntiles; ++t) {
    const int b = t & 1;
    if (!all_in && t + 1 < ntiles) issue(t + 1, b ^ 1);
    const unsigned char* kvs = L.kv[b];
    const int* rowok = L.rowok[b];

    // S^T: rows (4g+i) and (16+4g+i) against head `head`, four accumulator chains; lane
    // (g, col) reads chunk 4 ks + g of rows col and 16 + col (same swizzle)
    // (chunk 4 ks + g sits at 4 ks + (g ^ swz): one lane offset, the step is an immediate)
    const unsigned char* ra0 = kvs + col * kKvRowD + (g ^ kv_swz(col)) * 16;
    f32x4_t S0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, S1 = S0, S2 = S0, S3 = S0;
#pragma unroll
    for (int ks = 0; ks < 16; ks += 2) {
      const bf16x8_t A0 = *reinterpret_cast<const bf16x8_t*>(ra0 + ks * 64);
      const bf16x8_t A1 = *reinterpret_cast<const bf16x8_t*>(ra0 + 16 * kKvRowD + ks * 64);
      const bf16x8_t A2 = *reinterpret_cast<const bf16x8_t*>(ra0 + ks * 64 + 64);
      const bf16x8_t A3 = *reinterpret_cast<const bf16x8_t*>(ra0 + 16 * kKvRowD + ks * 64 + 64);
      S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, Qf[ks], S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, Qf[ks], S1, 0, 0, 0);
      S2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A2, Qf[ks + 1], S2, 0, 0, 0);
      S3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A3, Qf[ks + 1], S3, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) { S0[i] += S2[i]; S1[i] += S3[i]; }
    float s[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = rowok[4 * g + i] ? S0[i] * sl2 : neg_inf();
      s[4 + i] = rowok[16 + 4 * g + i] ? S1[i] * sl2 : neg_inf();
    }
    float tmax = s[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, s[i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    // The running maximum moves only when some head's tile maximum exceeds it by more than
    // kLazyMax (log2 units); below that p = 2^(s - m_run) <= 2^kLazyMax stays well inside the
    // fp32 and bf16 ranges and the output needs no rescale: the wave skips its 128 products.
    // Exact up to rounding: the sum and the output share the same m_run.
    const bool move = __builtin_amdgcn_ballot_w64(tmax > m_run + kLazyMax) != 0;
    const float m_new = move ? fmaxf(m_run, tmax) : m_run;
    const float alpha = (m_new == neg_inf() || m_new == m_run) ? 1.f : exp2f(m_run - m_new);
    float p[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = (s[i] == neg_inf()) ? 0.f : exp2f(s[i] - m_new);
      psum += p[i];
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // P as the A operand: row = head `col`, K slots (g, i) <-> rows {4g..4g+3, 16+4g..16+4g+3}
    bf16x8_t Pf;
#pragma unroll
    for (int i = 0; i < 8; ++i) Pf[i] = (__bf16)p[i];
    if (move) {
      float ai[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
      for (int nt = 0; nt < 32; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[nt][i] *= ai[i];
    }
    // V operand: slots 0-3 rows 4g .. 4g+3, slots 4-7 rows 16+4g .. 16+4g+3 of dim 16 nt + col;
    // this lane supplies row 4g + (col >> 2) (+16), dims 16 nt + 4 (col & 3) .. + 3: chunk
    // 2 nt + ((col & 3) >> 1), half col & 1
    // (chunk 2 nt + q sits at 2 nt + (q ^ swz): one lane offset, the step is an immediate)
    const int vrow = 4 * g + (col >> 2);   // rows vrow and vrow + 16 share the swizzle
    const unsigned char* vb0 =
        kvs + vrow * kKvRowD + (col & 1) * 8 + (((col & 3) >> 1) ^ kv_swz(vrow)) * 16;
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) {
      const unsigned char* vb = vb0 + nt * 32;
      const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s_t*)(vb));
      const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s_t*)(vb + 16 * kKvRowD));
      const v4s_t v8[2] = {lo, hi};
      const bf16x8_t Vf = *reinterpret_cast<const bf16x8_t*>(v8);
      O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Pf, Vf, O[nt], 0, 0, 0);
    }
    if (!all_in) {   // uniform
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (t + 1 < ntiles) expand(b ^ 1);
      __syncthreads();
    }
  }

  if (nsplit == 1) {
    const float zs = a.sink ? a.sink[head] * kLog2e : neg_inf();
    const float M = fmaxf(m_run, zs);
    float f = 0.f;
    if (M != neg_inf()) {
      const float em = (m_run == neg_inf()) ? 0.f : exp2f(m_run - M);
      const float den = l_run * em + ((zs == neg_inf()) ? 0.f : exp2f(zs - M));
      f = den > 0.f ? em / den : 0.f;
    }
    float fi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fi[i] = __shfl(f, 4 * g + i);
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + (r * kAH + 16 * wave) * kAD;
    const int rope0 = a.out_rope_dim > 0 ? kAD - a.out_rope_dim : kAD;
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) {
      float cs = 1.f, sn = 0.f;
      if (nt * 16 >= rope0)
        rope_cos_sin(-double(a.q_pos[r]), (nt * 16 + col - rope0) >> 1, a.out_rope_dim,
                     a.rope_log2_base, cs, sn);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float y = O[nt][i] * fi[i];
        if (nt * 16 >= rope0) y = rope_pair_lane(y, (col & 1) != 0, cs, sn);
        op[(4 * g + i) * kAD + nt * 16 + col] = f32_to_bf16(y);
      }
    }
  } else {
    const int64_t rs = r * nsplit + split;
    uint2* pp = part_out(a.ws, rs) + wave * 32 * kWave + lane;
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) pp[nt * kWave] = pack_bf16x4(O[nt]);
    if (g == 0) part_ml(a.ws, n_rows_total * nsplit, rs)[head] = make_float2(m_run, l_run);
  }
}

}  // namespace csa
