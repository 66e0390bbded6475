// Lightning-indexer scores on gfx950.
//
// score[r][s] = sum_j w[r][j] * ReLU(q[r][j] . k[s])   ("Lecture 10 - Hybrid
// LLMs", section 5.1, the indexer equation: few heads, low dimension, one key
// per position shared by every index head; FP8-friendly).
//
// BF16 / FP8 inputs run on MFMA with the heads on the M axis and 16 cache
// entries on the N axis of a 16x16x32 tile, so one key row feeds every head;
// the ReLU and the weighted head sum are an fp32 epilogue on the accumulator
// (4 heads per lane, then two cross-lane adds).  Full mode streams the
// visible entries of each row; candidate mode (Reindex, "CSA, HCA and CSA2",
// section 3.2) gathers the listed entries.  F32 inputs use a plain FMA kernel.
#include "kernels.hpp"

namespace sa {

namespace {

constexpr int kWaves = 4;  // waves per workgroup

template <bool FP8>
struct ElemTraits;
template <>
struct ElemTraits<false> {  // bf16
  static constexpr int bytes = 2;
};
template <>
struct ElemTraits<true> {  // OCP e4m3
  static constexpr int bytes = 1;
};

// One lane's slice of a key or query row for the MFMA: lane group g = lane/16
// holds the 16-byte pieces [64 i + 16 g, 64 i + 16 g + 16) of the row, so one
// load instruction reads 64 contiguous bytes of each of its 16 rows; k-step
// ks uses the lane's ks-th 8 elements.  Keys and queries share the mapping,
// so every k-step contracts the same channel set on both operands.
template <int DIM, bool FP8>
struct LaneSlice {
  static constexpr int KS = DIM / 32;
  static constexpr int BYTES = DIM / 4 * ElemTraits<FP8>::bytes;
  static constexpr int VEC = BYTES / 16;  // 16-byte vectors per lane
  u32x4 v[VEC];

  __device__ __forceinline__ void load(const char* row, int g) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row);
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = __builtin_nontemporal_load(p + 4 * i + g);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = u32x4{0, 0, 0, 0};
  }
};

template <int DIM>
__device__ __forceinline__ f32x4 mfma_slice(const LaneSlice<DIM, false>& a,
                                            const LaneSlice<DIM, false>& b, f32x4 acc) {
#pragma unroll
  for (int ks = 0; ks < LaneSlice<DIM, false>::KS; ++ks)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v[ks]),
                                                  __builtin_bit_cast(bf16x8, b.v[ks]), acc, 0, 0,
                                                  0);
  return acc;
}

template <int DIM>
__device__ __forceinline__ f32x4 mfma_slice(const LaneSlice<DIM, true>& a,
                                            const LaneSlice<DIM, true>& b, f32x4 acc) {
#pragma unroll
  for (int ks = 0; ks < LaneSlice<DIM, true>::KS; ++ks) {
    const uint32_t* pa = reinterpret_cast<const uint32_t*>(&a.v[0]) + 2 * ks;
    const uint32_t* pb = reinterpret_cast<const uint32_t*>(&b.v[0]) + 2 * ks;
    long la = (long)(((uint64_t)pa[1] << 32) | pa[0]);
    long lb = (long)(((uint64_t)pb[1] << 32) | pb[0]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(la, lb, acc, 0, 0, 0);
  }
  return acc;
}

// acc[t][mt] += Q[mt] . K[t] for NT key tiles, k-step
// outermost so the 4*NMT accumulator chains interleave.
template <int NMT, int DIM, int NT>
__device__ __forceinline__ void mfma_tiles(const LaneSlice<DIM, false> (&q)[NMT],
                                           const LaneSlice<DIM, false> (&k)[NT], f32x4 (&acc)[NT][NMT]) {
#pragma unroll
  for (int ks = 0; ks < LaneSlice<DIM, false>::KS; ++ks)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
        acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, q[mt].v[ks]), __builtin_bit_cast(bf16x8, k[t].v[ks]),
            acc[t][mt], 0, 0, 0);
}
template <int NMT, int DIM, int NT>
__device__ __forceinline__ void mfma_tiles(const LaneSlice<DIM, true> (&q)[NMT],
                                           const LaneSlice<DIM, true> (&k)[NT], f32x4 (&acc)[NT][NMT]) {
#pragma unroll
  for (int ks = 0; ks < LaneSlice<DIM, true>::KS; ++ks)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const uint32_t* pa = reinterpret_cast<const uint32_t*>(&q[mt].v[0]) + 2 * ks;
        const uint32_t* pb = reinterpret_cast<const uint32_t*>(&k[t].v[0]) + 2 * ks;
        const long la = (long)(((uint64_t)pa[1] << 32) | pa[0]);
        const long lb = (long)(((uint64_t)pb[1] << 32) | pb[0]);
        acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(la, lb, acc[t][mt], 0, 0, 0);
      }
}

// grid = (ceil(n_slots / (64*kWaves*gpw)), R); wave w scores gpw groups of 64
// consecutive slots of row blockIdx.y (gpw even), 16 entries per MFMA tile.
// The query slices and head weights are loaded once per wave; key rows
// stream through a two-deep register pipeline (the next group's rows load
// while the current group is scored).  Loads are unconditional, with the
// entry clamped to a visible one.
template <int DIM, bool FP8>
struct Group {
  LaneSlice<DIM, FP8> ks[4];
  int pos[4];
};

template <int NMT, int DIM, bool FP8, bool STAGED>
__global__ __launch_bounds__(64 * kWaves) void index_score_mfma(IndexArgs a, int gpw) {
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const RowInfo ri = row_info(a.rows, r);
  const bool cand_mode = a.cand != nullptr;
  const int n_slots = cand_mode ? a.cand_count[r] : ri.n_avail;
  const int wg_base = blockIdx.x * (64 * kWaves * gpw);
  if (wg_base >= n_slots) return;
  float* out = a.scores + (int64_t)r * a.score_stride;
  // nothing visible: every listed candidate scores -inf; dense route (at
  // most skip_k candidates, all of which any top-k with k >= skip_k keeps):
  // 0 for every visible entry, without reading the cache
  const bool dense_route = !cand_mode && a.skip_k > 0 && ri.win_lo <= a.skip_k;
  if (ri.n_avail == 0 || dense_route) {
    const float fill = dense_route ? 0.0f : -__builtin_huge_valf();
    for (int i = threadIdx.x; i < 64 * kWaves * gpw && wg_base + i < n_slots; i += 64 * kWaves)
      out[wg_base + i] = fill;
    return;
  }
  const int32_t* cand = cand_mode ? a.cand + (int64_t)r * a.cand_stride : nullptr;
  const int wbase = wg_base + wave * 64 * gpw;
  const int ngrp = min(gpw, (n_slots - wbase + 63) / 64);  // groups of this wave
  if (ngrp <= 0) return;

  // Without a candidate list, a group's 64 slots are consecutive; when the
  // cache's pages (a contiguous cache: one page per sequence) hold whole
  // groups, the group lies in one page.  The pages of all the wave's groups
  // are read up front with one vector load (lane i: group i's page, ngrp <=
  // 16), before any key load, and each group takes its page with a lane
  // read: no table load waits in the loop.  Slots past the row stay inside
  // that page.
  const bool page_per_group = !cand_mode && a.k.page_shift >= 6;
  const int wbase_u = __builtin_amdgcn_readfirstlane(wbase);
  int pg_lane = 0;
  if (page_per_group) {
    const int gl = lane < ngrp ? lane : 0;
    const int64_t lp = (int64_t)ri.b * a.k.max_pages + ((wbase_u + 64 * gl) >> a.k.page_shift);
    pg_lane = a.k.block_table ? a.k.block_table[lp] : (int)lp;
  }
  auto load_group = [&](int gi, Group<DIM, FP8>& G) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int slot = wbase + 64 * gi + 16 * t + col;
      G.pos[t] = cand_mode ? cand[min(slot, n_slots - 1)] : slot;
    }
    if (page_per_group) {
      const int s0 = wbase_u + 64 * gi;
      const int64_t page = __builtin_amdgcn_readlane(pg_lane, gi);
      const char* pbase = a.k.data + page * a.k.page_size * a.k.row_stride;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int off = (s0 + 16 * t + col) & (a.k.page_size - 1);
        G.ks[t].load(pbase + (int64_t)off * a.k.row_stride, g);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int pc = min(max(G.pos[t], 0), ri.n_avail - 1);
        G.ks[t].load(cache_row(a.k, ri.b, pc), g);
      }
    }
  };
  // Rows stored back to back (one page holds the group as 64 contiguous
  // rows): load the group in 8 KB units, each as eight 1 KB wave-contiguous
  // pieces (whole cache lines per instruction; the MFMA lane layout would
  // read sixteen half lines per instruction, about 15% slower from HBM), and
  // reshape each unit through a wave-private LDS tile (rows padded by 16
  // bytes: the MFMA-layout reads are then free of bank conflicts).
  // (STAGED: the host checked every condition: pages of whole groups, rows
  // of 128 or 256 bytes back to back, no candidate list)
  constexpr int ROWB = DIM * ElemTraits<FP8>::bytes;
  static_assert(!STAGED || ROWB == 128 || ROWB == 256, "staged rows are 128 or 256 bytes");
  constexpr bool staged = STAGED;
  constexpr int UNITS = ROWB >= 128 ? ROWB / 128 : 1;  // 8 KB units per group
  constexpr int RU = 64 / UNITS;     // rows per unit
  constexpr int PPR = ROWB / 16;     // 16-byte pieces per row
  constexpr int TPU = 4 / UNITS;     // MFMA tiles per unit
  u32x4 raw[8];
  auto load_raw = [&](int gi, int un) {
    const int s0 = wbase_u + 64 * gi;
    const int64_t page = __builtin_amdgcn_readlane(pg_lane, gi);
    const u32x4* gb = reinterpret_cast<const u32x4*>(
        a.k.data + (page * a.k.page_size + (s0 & (a.k.page_size - 1))) * (int64_t)ROWB + 8192 * un);
#pragma unroll
    for (int u = 0; u < 8; ++u) raw[u] = __builtin_nontemporal_load(gb + 64 * u + lane);
  };
  Group<DIM, FP8> buf[2];
  if constexpr (staged)
    load_raw(0, 0);
  else
    load_group(0, buf[0]);

  // Query slices (A operand: head = mt*16 + col) and head weights in the
  // accumulator layout (head = mt*16 + 4*g + i).
  constexpr int EB = ElemTraits<FP8>::bytes;
  LaneSlice<DIM, FP8> qs[NMT];
  float wv[NMT][4];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int h = mt * 16 + col;
    if (h < a.n_heads)
      qs[mt].load(reinterpret_cast<const char*>(a.q) + ((int64_t)r * a.n_heads + h) * DIM * EB, g);
    else
      qs[mt].zero();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hw = mt * 16 + 4 * g + i;
      wv[mt][i] = hw < a.n_heads ? a.w[(int64_t)r * a.n_heads + hw] : 0.0f;
    }
  }

  // The four tiles' MFMA chains and epilogues are independent: interleave
  // them (k-step outermost) so the chains overlap.
  auto epilogue = [&](int gi, const f32x4 (&acc)[4][NMT], const int (&pos)[4]) {
    const int base = wbase + 64 * gi;
    float res[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float part[4] = {0.f, 0.f, 0.f, 0.f};  // one chain per accumulator row
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[i] = fmaf(wv[mt][i], relu(acc[t][mt][i]), part[i]);
      res[t] = (part[0] + part[1]) + (part[2] + part[3]);
    }
    // lane l stores the result of slot base + l (tile l/16, column l%16)
    const float sum = sum4_transposed(res[0], res[1], res[2], res[3]);  // all lanes take part
    // validity of tile t's column as bit t (a lane-dependent pick from G.pos
    // would put the whole group in scratch memory)
    unsigned vb = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) vb |= (unsigned)(pos[t] >= 0 && pos[t] < ri.n_avail) << t;
    if (base + lane < n_slots) out[base + lane] = (vb >> g) & 1u ? sum : -__builtin_huge_valf();
  };
  auto score_group = [&](int gi, const Group<DIM, FP8>& G) {
    f32x4 acc[4][NMT];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    mfma_tiles<NMT, DIM, 4>(qs, G.ks, acc);
    epilogue(gi, acc, G.pos);
  };

  if constexpr (staged) {
    __shared__ u32x4 stage[kWaves][RU][PPR + 1];
    u32x4(&tile)[RU][PPR + 1] = stage[wave];
    for (int gi = 0; gi < ngrp; ++gi) {
      f32x4 acc[4][NMT];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int un = 0; un < UNITS; ++un) {
        // The tile passes rows between lanes of the wave: LDS runs a wave's
        // accesses in order, so only the compiler must keep them in program
        // order (it would otherwise move the reads above the other lanes'
        // writes, or the next unit's writes above these reads).
        asm volatile("" ::: "memory");
#pragma unroll
        for (int u = 0; u < 8; ++u) tile[(64 * u + lane) / PPR][(64 * u + lane) % PPR] = raw[u];
        asm volatile("" ::: "memory");
        if (un + 1 < UNITS)
          load_raw(gi, un + 1);
        else if (gi + 1 < ngrp)
          load_raw(gi + 1, 0);
        LaneSlice<DIM, FP8> ks[TPU];
#pragma unroll
        for (int tl = 0; tl < TPU; ++tl)
#pragma unroll
          for (int i = 0; i < LaneSlice<DIM, FP8>::VEC; ++i) ks[tl].v[i] = tile[16 * tl + col][4 * i + g];
        asm volatile("" ::: "memory");
        mfma_tiles<NMT, DIM, TPU>(qs, ks, *reinterpret_cast<f32x4(*)[TPU][NMT]>(&acc[un * TPU]));
      }
      int pos[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) pos[t] = wbase + 64 * gi + 16 * t + col;
      epilogue(gi, acc, pos);
    }
  } else {
    // two groups per iteration so the buffer index stays static
    int gi = 0;
    for (; gi + 2 <= ngrp; gi += 2) {
      load_group(gi + 1, buf[1]);
      score_group(gi, buf[0]);
      if (gi + 2 < ngrp) load_group(gi + 2, buf[0]);
      score_group(gi + 1, buf[1]);
    }
    if (gi < ngrp) score_group(gi, buf[0]);
  }
}

// ----------------------------------------------------------------- prefill
// Many query rows of one sequence (prefill) make the score a GEMM: M = (query
// row, head), N = cache entries, K = dim.  A workgroup holds kPRowsW rows per
// wave (their FP8 query rows as the A operand of v_mfma_scale 16x16x128,
// heads on M, the whole 128-wide contraction in one instruction) and streams
// 64-entry chunks of the sequence's keys through LDS, shared by every row of
// the workgroup.  Blocks run heaviest (latest rows) first; a block whose rows
// span several sequences makes one pass per sequence.
constexpr int kPWaves = 8;
constexpr int kPRowsW = 1;                  // rows per wave
constexpr int kPRows = kPWaves * kPRowsW;   // rows per workgroup
constexpr int kPChunk = 64;                 // entries per LDS chunk
constexpr int kPTiles = kPChunk / 16;       // 16-entry MFMA tiles per chunk
constexpr int kPRowB = 128 + 16;            // LDS bytes per entry (padded)

typedef __attribute__((ext_vector_type(8))) int i32x8;

template <int NMT>
__global__ __launch_bounds__(64 * kPWaves) void index_score_prefill(IndexArgs a, int n_blocks) {
  __shared__ __align__(16) char kb[2][kPChunk * kPRowB];
  __shared__ int sb[kPRows], sn[kPRows], sz[kPRows];
  __shared__ int wred[kPWaves][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int r0 = (n_blocks - 1 - (int)blockIdx.x) * kPRows;
  if (tid < kPRows) {
    const int r = r0 + tid;
    int b = -1, n = 0, zero = 0;
    if (r < a.rows.n_rows) {
      const RowInfo ri = row_info(a.rows, r);
      b = ri.b;
      n = ri.n_avail;
      // dense route: a row whose candidates all fit the budget gets zeros
      if (b >= 0 && a.skip_k > 0 && ri.win_lo <= a.skip_k) {
        zero = n;
        n = 0;
      }
    }
    sb[tid] = b;
    sn[tid] = b >= 0 ? n : 0;
    sz[tid] = zero;
  }
  __syncthreads();
  for (int j = 0; j < kPRows; ++j)
    for (int i = tid; i < sz[j]; i += 64 * kPWaves)
      a.scores[(int64_t)(r0 + j) * a.score_stride + i] = 0.0f;

  // this wave's rows: A operands (head mt*16 + col, bytes [32g, 32g+32)) and
  // head weights in the accumulator layout (head mt*16 + 4g + i)
  i32x8 qa[kPRowsW][NMT];
  float wv[kPRowsW][NMT][4];
  int rb[kPRowsW], rn[kPRowsW];
#pragma unroll
  for (int j = 0; j < kPRowsW; ++j) {
    const int lr = wave * kPRowsW + j, r = r0 + lr;
    rb[j] = sb[lr];
    rn[j] = sn[lr];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int h = mt * 16 + col;
      if (rb[j] >= 0 && h < a.n_heads) {
        const u32x4* qp = reinterpret_cast<const u32x4*>(
            reinterpret_cast<const char*>(a.q) + ((int64_t)r * a.n_heads + h) * 128 + 32 * g);
        const u32x4 x0 = qp[0], x1 = qp[1];
        qa[j][mt] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                          (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
      } else {
        qa[j][mt] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hw = mt * 16 + 4 * g + i;
        wv[j][mt][i] = (rb[j] >= 0 && hw < a.n_heads) ? a.w[(int64_t)r * a.n_heads + hw] : 0.0f;
      }
    }
  }

  // one pass per distinct sequence of the block, in increasing order
  int bprev = -1;
  while (true) {
    int bs = 0x7FFFFFFF, nmax = 0;
    for (int i = 0; i < kPRows; ++i)
      if (sb[i] > bprev) bs = min(bs, sb[i]);
    if (bs == 0x7FFFFFFF) break;
    for (int i = 0; i < kPRows; ++i)
      if (sb[i] == bs) nmax = max(nmax, sn[i]);
    bprev = bs;
    if (nmax == 0) continue;

    // chunk loads: piece p = tid + i*blockDim is entry p/8 of the chunk,
    // 16 bytes at 16 (p%8)
    constexpr int PPT = kPChunk * 8 / (64 * kPWaves);
    static_assert(PPT * 64 * kPWaves == kPChunk * 8, "whole 16-byte pieces per thread");
    u32x4 pre[PPT];
    auto load_chunk = [&](int c0) {
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int pc = tid + i * 64 * kPWaves;
        const int e = min(c0 + (pc >> 3), nmax - 1);
        pre[i] = *reinterpret_cast<const u32x4*>(cache_row(a.k, bs, e) + 16 * (pc & 7));
      }
    };
    load_chunk(0);
    int buf = 0;
    for (int c0 = 0; c0 < nmax; c0 += kPChunk) {
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int pc = tid + i * 64 * kPWaves;
        *reinterpret_cast<u32x4*>(&kb[buf][(pc >> 3) * kPRowB + 16 * (pc & 7)]) = pre[i];
      }
      __syncthreads();
      if (c0 + kPChunk < nmax) load_chunk(c0 + kPChunk);
      // Tile t+1's MFMAs are issued before tile t's epilogue, so the matrix
      // pipe works while the VALU applies ReLU and the head weights.
      float res[kPRowsW][4];  // lane partial of each of the last 4 tiles
      f32x4 acc[2][kPRowsW][NMT];
      auto issue = [&](int t, f32x4 (&A)[kPRowsW][NMT]) {
        const char* kr = &kb[buf][(16 * t + col) * kPRowB + 32 * g];
        const u32x4 y0 = *reinterpret_cast<const u32x4*>(kr);
        const u32x4 y1 = *reinterpret_cast<const u32x4*>(kr + 16);
        const i32x8 kbv = {(int)y0[0], (int)y0[1], (int)y0[2], (int)y0[3],
                           (int)y1[0], (int)y1[1], (int)y1[2], (int)y1[3]};
#pragma unroll
        for (int j = 0; j < kPRowsW; ++j)
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt)
            A[j][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                qa[j][mt], kbv, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0x7F7F7F7F, 0, 0x7F7F7F7F);
      };
      auto epilogue = [&](int t, const f32x4 (&A)[kPRowsW][NMT]) {
#pragma unroll
        for (int j = 0; j < kPRowsW; ++j) {
          // one fma chain: the tiles in flight and the waves sharing the
          // SIMD cover its latency, and no adds are needed to join chains
          float part = 0.f;
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) part = fmaf(wv[j][mt][i], relu(A[j][mt][i]), part);
          res[j][t & 3] = part;
        }
        // After every 4 tiles, one transposed reduction over the four lane
        // groups leaves lane l with entry l of those 64 (tile l/16, column
        // l%16).
        if ((t & 3) == 3) {
#pragma unroll
          for (int j = 0; j < kPRowsW; ++j) {
            const float mine = sum4_transposed(res[j][0], res[j][1], res[j][2], res[j][3]);
            const int e = c0 + 16 * (t - 3) + lane;
            if (rb[j] == bs && e < rn[j])
              a.scores[(int64_t)(r0 + wave * kPRowsW + j) * a.score_stride + e] = mine;
          }
        }
      };
      static_assert(kPTiles % 4 == 0, "whole 64-entry store groups per chunk");
      issue(0, acc[0]);
#pragma unroll
      for (int t = 0; t < kPTiles; t += 2) {
        issue(t + 1, acc[1]);
        epilogue(t, acc[0]);
        if (t + 2 < kPTiles) issue(t + 2, acc[0]);
        epilogue(t + 1, acc[1]);
      }
      // No barrier here: the next chunk is stored into the other buffer,
      // whose last readers (the previous chunk) all passed this chunk's
      // barrier.
      buf ^= 1;
    }
  }
}

// F32 path: one thread per (row, slot); the row's query and weights in LDS.
__global__ __launch_bounds__(256) void index_score_f32(IndexArgs a) {
  extern __shared__ float smem[];
  const int r = blockIdx.y;
  const RowInfo ri = row_info(a.rows, r);
  const bool cand_mode = a.cand != nullptr;
  const int n_slots = cand_mode ? a.cand_count[r] : ri.n_avail;
  const int slot = blockIdx.x * blockDim.x + threadIdx.x;
  if ((int)(blockIdx.x * blockDim.x) >= n_slots) return;
  const int HD = a.n_heads * a.dim;
  const float* q = reinterpret_cast<const float*>(a.q) + (int64_t)r * HD;
  for (int i = threadIdx.x; i < HD; i += blockDim.x) smem[i] = q[i];
  for (int i = threadIdx.x; i < a.n_heads; i += blockDim.x) smem[HD + i] = a.w[(int64_t)r * a.n_heads + i];
  __syncthreads();
  if (slot >= n_slots) return;
  int pos = cand_mode ? a.cand[(int64_t)r * a.cand_stride + slot] : slot;
  float s = -__builtin_huge_valf();
  if (!cand_mode && a.skip_k > 0 && ri.win_lo <= a.skip_k) {
    s = 0.0f;  // dense route: every candidate is kept whatever its score
  } else if (pos >= 0 && pos < ri.n_avail) {
    const float* kr = reinterpret_cast<const float*>(cache_row(a.k, ri.b, pos));
    s = 0.0f;
    for (int h = 0; h < a.n_heads; ++h) {
      float d = 0.0f;
      for (int c = 0; c < a.dim; ++c) d = fmaf(smem[h * a.dim + c], kr[c], d);
      s = fmaf(smem[HD + h], relu(d), s);
    }
  }
  a.scores[(int64_t)r * a.score_stride + slot] = s;
}

template <int NMT, int DIM, bool FP8>
hipError_t launch_mfma(const IndexArgs& a, hipStream_t s) {
  // Enough workgroups to cover the 256 CUs several times; long rows give each
  // wave more 64-entry groups, so the query load is amortised over them.
  const int per_group = 64 * kWaves;
  const int groups = (a.n_slots + per_group - 1) / per_group;
  int gpw = 2;
  while (gpw < 16 && (int64_t)((groups + 2 * gpw - 1) / (2 * gpw)) * a.rows.n_rows >= 1024) gpw *= 2;
  dim3 grid((groups + gpw - 1) / gpw, a.rows.n_rows);
  constexpr int rowb = DIM * (FP8 ? 1 : 2);
  constexpr bool stageable = rowb == 128 || rowb == 256;
  const bool staged = stageable && a.cand == nullptr && a.k.page_shift >= 6 && a.k.row_stride == rowb;
  if (staged)
    hipLaunchKernelGGL((index_score_mfma<NMT, DIM, FP8, stageable>), grid, dim3(64 * kWaves), 0, s, a, gpw);
  else
    hipLaunchKernelGGL((index_score_mfma<NMT, DIM, FP8, false>), grid, dim3(64 * kWaves), 0, s, a, gpw);
  return hipGetLastError();
}

template <int DIM, bool FP8>
hipError_t dispatch_heads(const IndexArgs& a, hipStream_t s) {
  if (a.n_heads <= 16) return launch_mfma<1, DIM, FP8>(a, s);
  if (a.n_heads <= 32) return launch_mfma<2, DIM, FP8>(a, s);
  return launch_mfma<4, DIM, FP8>(a, s);
}

}  // namespace

// Host dispatch.  Shapes are validated by the ABI layer: BF16 / FP8 need
// dim in {64, 128} and at most 64 heads.
hipError_t launch_index_score(const IndexArgs& a, hipStream_t s) {
  if (a.rows.n_rows == 0 || a.n_slots == 0) return hipSuccess;
  if (a.dtype == 0) {
    dim3 grid((a.n_slots + 255) / 256, a.rows.n_rows);
    size_t lds = sizeof(float) * (size_t)(a.n_heads * a.dim + a.n_heads);
    hipLaunchKernelGGL(index_score_f32, grid, dim3(256), lds, s, a);
    return hipGetLastError();
  }
  const bool fp8 = a.dtype == 2;
  // Many rows of FP8 128-wide keys (prefill): the GEMM-shaped kernel.
  if (fp8 && a.dim == 128 && a.cand == nullptr && a.rows.n_rows >= kPRows && a.n_heads <= 64) {
    const int n_blocks = (a.rows.n_rows + kPRows - 1) / kPRows;
    const int nmt = (a.n_heads + 15) / 16;
    if (nmt == 4)
      hipLaunchKernelGGL(index_score_prefill<4>, dim3(n_blocks), dim3(64 * kPWaves), 0, s, a, n_blocks);
    else if (nmt == 2)
      hipLaunchKernelGGL(index_score_prefill<2>, dim3(n_blocks), dim3(64 * kPWaves), 0, s, a, n_blocks);
    else if (nmt == 3)
      hipLaunchKernelGGL(index_score_prefill<3>, dim3(n_blocks), dim3(64 * kPWaves), 0, s, a, n_blocks);
    else
      hipLaunchKernelGGL(index_score_prefill<1>, dim3(n_blocks), dim3(64 * kPWaves), 0, s, a, n_blocks);
    return hipGetLastError();
  }
  if (a.dim == 64) return fp8 ? dispatch_heads<64, true>(a, s) : dispatch_heads<64, false>(a, s);
  return fp8 ? dispatch_heads<128, true>(a, s) : dispatch_heads<128, false>(a, s);
}

}  // namespace sa
