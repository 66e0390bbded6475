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
// consecutive slots of row blockIdx.y, 16 entries per MFMA tile.
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
// row, head), N = cache entries, K = dim.  A workgroup holds one row per wave
// (its FP8 query as the A operand of v_mfma_scale 16x16x128, heads on M, the
// whole 128-wide contraction in one instruction) and streams 64-entry chunks
// of the sequence's keys through LDS, shared by every row of the workgroup.
// Blocks run heaviest (latest rows) first; a block whose rows span several
// sequences makes one pass per sequence.
//
// The epilogue is where the time goes: every (head, entry) product needs a
// ReLU and a weighted add on the VALU while the matrix pipe does 128 MACs.
// With ReLU(x) = (x + |x|) / 2,
//   sum_h w_h ReLU(s_h) = 1/2 sum_h w_h |s_h| + 1/2 (sum_h w_h q_h) . k,
// and the first half is one fma per product (|x| is a free source
// modifier).  The second half is linear in the key, so the MFMA takes it:
// q' = sum_h w_h q_h (fp32, per row) is split into kLimbs FP8 rows
// q' = sum_j 2^e(j,b) c_j (each limb takes the next ~4 significant bits of
// what the previous ones left, with one E8M0 scale per limb and 32-channel
// block b), which fill rows 4i and 4i+1 of one more 16-row A tile.  Its
// accumulator rows sum to q'.k / 2 (the 1/2 rides in the scales), so each
// lane starts its fma chain with its two limb rows and the transposed
// reduction does the rest.  On integer
// inputs q' is an exact integer, every limb decodes to integers and every
// partial sum stays below 2^24, so the scores are exact.
constexpr int kPWaves = 8;
constexpr int kPRows = kPWaves;             // rows per workgroup, one per wave
constexpr int kPChunk = 64;                 // entries per LDS chunk
constexpr int kPPT = kPChunk * 8 / (64 * kPWaves);  // 16-byte pieces per thread per chunk
constexpr int kPTiles = kPChunk / 16;       // 16-entry MFMA tiles per chunk
constexpr int kPRowB = 128;                 // LDS bytes per entry
// LDS swizzle: 16-byte piece j of entry e sits in slot j ^ ((e >> 1) & 7) of
// its row, so 16 lanes reading one piece of 16 consecutive entries, or
// writing two whole entries, touch 16 distinct 16-byte bank groups.
__device__ __forceinline__ int kslot(int e, int j) { return 16 * (j ^ ((e >> 1) & 7)); }
constexpr int kLimbs = 8;                   // FP8 limbs of q' (about 32 bits), two per lane group
constexpr int kPMaxSub = 1024;              // 64-entry pieces per pass with a block table
// Word 3 of a raw buffer resource on CDNA (32-bit dword accesses,
// range-checked against the resource's byte size: stores past it are
// dropped).
constexpr int kOutWord3 = 0x00020000;

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(2))) float f32x2;
struct Pre {
  u32x4 v[kPPT];
};

__device__ __forceinline__ i32x8 cat8(u32x4 x0, u32x4 x1) {
  return i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
               (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
}

template <int NMT, bool TABLE>
__global__ __launch_bounds__(64 * kPWaves) void index_score_prefill(IndexArgs a, int n_blocks) {
  __shared__ __align__(16) char kb[2][kPChunk * kPRowB];
  __shared__ __align__(16) uint8_t limb[kPWaves][16 * 128];  // [wave][limb row][channel]
  __shared__ uint8_t limb_scale[kPWaves][16 * 4];            // [wave][limb row][block]
  __shared__ int sb[kPRows], sn[kPRows], sz[kPRows];
  __shared__ int cpage[TABLE ? kPMaxSub : 1];  // page of each 64-entry piece of the pass
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

  // This wave's row: A operands (head mt*16 + col, bytes [32g, 32g+32)) and
  // half the head weights in the accumulator layout (head mt*16 + 4g + i).
  const int r = __builtin_amdgcn_readfirstlane(r0 + wave);
  const int rb = __builtin_amdgcn_readfirstlane(sb[wave]);
  const int rn = __builtin_amdgcn_readfirstlane(sn[wave]);
  i32x8 qa[NMT];
  float wh[NMT][4];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int h = mt * 16 + col;
    if (rb >= 0 && h < a.n_heads) {
      const u32x4* qp = reinterpret_cast<const u32x4*>(
          reinterpret_cast<const char*>(a.q) + ((int64_t)r * a.n_heads + h) * 128 + 32 * g);
      qa[mt] = cat8(qp[0], qp[1]);
    } else {
      qa[mt] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hw = mt * 16 + 4 * g + i;
      wh[mt][i] = (rb >= 0 && hw < a.n_heads) ? 0.5f * a.w[(int64_t)r * a.n_heads + hw] : 0.0f;
    }
  }

  // q' = sum_h w_h q_h; lane l owns channels 2l and 2l + 1.
  float x0 = 0.f, x1 = 0.f;
  if (rb >= 0) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(
                             reinterpret_cast<const char*>(a.q) + (int64_t)r * a.n_heads * 128) + lane;
    const float* wr = a.w + (int64_t)r * a.n_heads;
#pragma unroll 8
    for (int h = 0; h < a.n_heads; ++h) {
      const f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)qp[64 * h], false);
      const float w = wr[h];
      x0 = fmaf(w, f.x, x0);
      x1 = fmaf(w, f.y, x1);
    }
  }
  // Limbs: each takes what the previous ones left, rounded to FP8 under a
  // power-of-two scale set by the largest remainder of its scale block.  A
  // limb that decodes to d leaves x - d exactly, so the limbs sum to q' up
  // to the last remainder.
  //
  // Scale blocks follow the matrix unit's K order, not the channel order: in
  // a 16x16x128 operand, bytes [0, 16) of lane group g are K [16g, 16g+16)
  // and bytes [16, 32) are K [64+16g, +16), and lane group b's scales cover
  // K [32b, 32b+32).  With lane group g holding channels [32g, 32g+32),
  // block 2h+p is channels {c : (c >> 4) & 1 == h, c >> 6 == p}: for
  // channels 2l and 2l+1, h is bit 3 of l and p is bit 5, and the 16 lanes
  // of a block differ in bits 0, 1, 2 and 4.
  const int blk = 2 * ((lane >> 3) & 1) + (lane >> 5);
  static_assert(kLimbs == 8, "rows 4i and 4i+1 of the tile");
#pragma unroll
  for (int j = 0; j < 16; ++j) {  // tile row j: limb 2 (j / 4) + j % 4 if j % 4 < 2
    uint32_t two = 0;
    int sc = 127;
    if (j % 4 < 2) {
      float m = fmaxf(fabsf(x0), fabsf(x1));
      m = fmaxf(m, __shfl_xor(m, 1));
      m = fmaxf(m, __shfl_xor(m, 2));
      m = fmaxf(m, __shfl_xor(m, 4));
      m = fmaxf(m, __shfl_xor(m, 16));
      if (m > 0.f) {
        // m < 2^E, so |x| * 2^-(E-8) < 256, inside FP8's range
        const int e = min(max(__builtin_amdgcn_frexp_expf(m) - 8, -126), 127);
        const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(x0, -e),
                                                       __builtin_amdgcn_ldexpf(x1, -e), 0, false);
        const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(pk, false);
        x0 -= __builtin_amdgcn_ldexpf(d.x, e);
        x1 -= __builtin_amdgcn_ldexpf(d.y, e);
        two = (uint32_t)pk & 0xFFFFu;
        sc = 126 + e;  // 2^(e-1): the 1/2 of the linear half
      }
    }
    *reinterpret_cast<uint16_t*>(&limb[wave][j * 128 + 2 * lane]) = (uint16_t)two;
    if ((lane & 0x17) == 0) limb_scale[wave][j * 4 + blk] = (uint8_t)sc;
  }
  __syncthreads();
  const i32x8 la = cat8(*reinterpret_cast<const u32x4*>(&limb[wave][col * 128 + 32 * g]),
                        *reinterpret_cast<const u32x4*>(&limb[wave][col * 128 + 32 * g + 16]));
  const int lsc = limb_scale[wave][col * 4 + g];  // lane (col, g): limb col, block g

  // one pass per distinct sequence of the block, in increasing order
  int bprev = -1;
  while (true) {
    int bs = 0x7FFFFFFF, nmax = 0;
    for (int i = 0; i < kPRows; ++i)
      if (sb[i] > bprev) bs = min(bs, sb[i]);
    if (bs == 0x7FFFFFFF) break;
    for (int i = 0; i < kPRows; ++i)
      if (sb[i] == bs) nmax = max(nmax, sn[i]);
    bs = __builtin_amdgcn_readfirstlane(bs);
    nmax = __builtin_amdgcn_readfirstlane(nmax);
    bprev = bs;
    if (nmax == 0) continue;
    // every wave is done with the previous pass's LDS (chunks, pages)
    __syncthreads();
    // With a block table, each chunk's page is read here once per pass and
    // kept in LDS: a table read inside the loop would be a vector load whose
    // wait also waits for the chunk loads in flight before it.
    const int nsub = (nmax + 63) / 64;  // 64-entry pieces: <= kPMaxSub (host check)
    if (TABLE) {
      for (int ci = tid; ci < min(nsub, kPMaxSub); ci += 64 * kPWaves)
        cpage[ci] = a.k.block_table[(int64_t)bs * a.k.max_pages + ((ci * 64) >> a.k.page_shift)];
      __syncthreads();
    }

    // chunk loads: thread tid fetches 16 bytes at 16 (tid % 8) of entries
    // tid / 8 + 64 i of the chunk (clamped to the last visible entry).  Each
    // 64-entry piece starts at a multiple of 64 and lies in one page (the
    // host sends a block table here only with pages of at least 64 entries),
    // so its first row comes from scalar arithmetic and each thread adds its
    // own offset.
    const int pe = tid >> 3, pb = 16 * (tid & 7);
    const int rs = (int)a.k.row_stride;  // at most 2^24 (host check)
    // Every chunk issues the same loads and stores, so the compiler's wait
    // counts stay exact across iterations: loads past the last chunk re-read
    // it, and the score stores are range-checked buffer stores (lanes past
    // the row, or every lane when the row is not in this pass, are dropped
    // by the hardware).
    const int last = (nmax - 1) & ~63;  // first entry of the last 64-entry piece
    auto load_chunk = [&](int c, Pre& pre) {
#pragma unroll
      for (int i = 0; i < kPPT; ++i) {
        // piece i: 64 entries from sub (in one page), clamped to the row
        const int sub = min(c + 64 * i, last);
        int64_t slot;
        if (TABLE) {
          const int pg = __builtin_amdgcn_readfirstlane(cpage[min(sub / 64, kPMaxSub - 1)]);
          slot = ((int64_t)pg << a.k.page_shift) + (sub & (a.k.page_size - 1));
        } else {
          slot = (int64_t)bs * a.k.max_pages * a.k.page_size + sub;
        }
        const uint32_t off = (uint32_t)(__mul24(min(pe, nmax - 1 - sub), rs) + pb);
        pre.v[i] = *reinterpret_cast<const u32x4*>(a.k.data + slot * a.k.row_stride + off);
      }
    };
    const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(
        a.scores + (int64_t)r * a.score_stride, (short)0, rb == bs ? 4 * rn : 0, kOutWord3);
    // One chunk: store its prefetched pieces, then (after the barrier) start
    // the loads of the chunk two ahead into the same registers, and score.
    auto chunk = [&](int c0, int buf, Pre& pre) {
#pragma unroll
      for (int i = 0; i < kPPT; ++i)
        *reinterpret_cast<u32x4*>(&kb[buf][(pe + 64 * i) * kPRowB + kslot(pe, tid & 7)]) = pre.v[i];
      __syncthreads();
      load_chunk(c0 + 2 * kPChunk, pre);
      // Tile t+1's MFMAs are issued before tile t's epilogue, so the matrix
      // pipe works while the VALU finishes the scores.
      float res[4];  // lane partial of each of the last 4 tiles
      f32x4 acc[2][NMT + 1];
      auto issue = [&](int t, f32x4 (&A)[NMT + 1]) {
        const char* kr = &kb[buf][(16 * t + col) * kPRowB];
        const i32x8 kbv = cat8(*reinterpret_cast<const u32x4*>(kr + kslot(col, 2 * g)),
                               *reinterpret_cast<const u32x4*>(kr + kslot(col, 2 * g + 1)));
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
          A[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              qa[mt], kbv, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0x7F7F7F7F, 0, 0x7F7F7F7F);
        A[NMT] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(la, kbv, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                                 lsc, 0, 0x7F7F7F7F);
      };
      auto epilogue = [&](int t, const f32x4 (&A)[NMT + 1]) {
        // the lane's two limb rows start one fma chain; the tiles in flight
        // and the waves sharing the SIMD cover its latency
        float part = A[NMT][0] + A[NMT][1];
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) part = fmaf(wh[mt][i], fabsf(A[mt][i]), part);
        res[t & 3] = part;
        if ((t & 3) == 3) {
          // one transposed reduction over the four lane groups leaves lane
          // l with entry 16 (t - 3) + l of the chunk (tile l/16, column l%16)
          const float mine = sum4_transposed(res[0], res[1], res[2], res[3]);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(mine), out, 4 * (c0 + 16 * (t - 3) + lane), 0, 0);
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
    };
    // Two chunks per iteration keep the prefetch registers static.  Chunk c
    // uses LDS buffer c % 2; it is stored again (chunk c + 2) only after the
    // barrier of chunk c + 1, which every wave reaches after scoring chunk c.
    // Stores that the hardware drops (a zero-size range) give the first
    // iteration the loop's own order of loads and stores, so the waits
    // before each LDS store can leave the other chunk's loads in flight.
    const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(a.scores, (short)0, 0, kOutWord3);
    Pre pre0, pre1;
    load_chunk(0, pre0);
#pragma unroll
    for (int i = 0; i < kPTiles / 4; ++i) __builtin_amdgcn_raw_buffer_store_b32(0u, none, 4 * i, 0, 0);
    load_chunk(kPChunk, pre1);
#pragma unroll
    for (int i = 0; i < kPTiles / 4; ++i) __builtin_amdgcn_raw_buffer_store_b32(0u, none, 64 + 4 * i, 0, 0);
    int c0 = 0;
    for (; c0 + kPChunk < nmax; c0 += 2 * kPChunk) {
      chunk(c0, 0, pre0);
      chunk(c0 + kPChunk, 1, pre1);
    }
    if (c0 < nmax) chunk(c0, 0, pre0);
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

template <bool TABLE>
hipError_t launch_prefill(const IndexArgs& a, int nmt, int n_blocks, hipStream_t s) {
  const dim3 grid(n_blocks), block(64 * kPWaves);
  if (nmt == 4)
    hipLaunchKernelGGL((index_score_prefill<4, TABLE>), grid, block, 0, s, a, n_blocks);
  else if (nmt == 3)
    hipLaunchKernelGGL((index_score_prefill<3, TABLE>), grid, block, 0, s, a, n_blocks);
  else if (nmt == 2)
    hipLaunchKernelGGL((index_score_prefill<2, TABLE>), grid, block, 0, s, a, n_blocks);
  else
    hipLaunchKernelGGL((index_score_prefill<1, TABLE>), grid, block, 0, s, a, n_blocks);
  return hipGetLastError();
}

// Workgroups of `kernel` (64 kWaves threads) that the whole GPU holds at
// once: the occupancy the registers and LDS allow per CU, times the CUs.
// Taken once per kernel (on the device current at the first call).
int resident_workgroups(const void* kernel) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * kWaves, 0) != hipSuccess)
    return 0;
  return max(cus, 1) * max(per_cu, 1);
}

// Groups per wave: each wave scores gpw 64-entry groups, one after another,
// so a launch takes about ceil(workgroups / resident) * gpw group times.
// Take the gpw in [2, 16] that minimises that (ties: the larger gpw, whose
// fewer workgroups load the queries fewer times).  A last partial round of
// long waves is what this avoids: 1024 workgroups of 8 groups per wave
// where 768 fit made the CSA2 Full indexer 103 against 94 us.
int pick_gpw(int groups, int rows, int resident) {
  if (resident <= 0) resident = 1024;
  int best = 2;
  int64_t best_cost = -1;
  for (int gpw = 2; gpw <= 16; ++gpw) {
    const int64_t wgs = (int64_t)((groups + gpw - 1) / gpw) * rows;
    const int64_t cost = (wgs + resident - 1) / resident * gpw;
    if (best_cost < 0 || cost <= best_cost) {
      best = gpw;
      best_cost = cost;
    }
  }
  return best;
}

template <int NMT, int DIM, bool FP8>
hipError_t launch_mfma(const IndexArgs& a, hipStream_t s) {
  const int per_group = 64 * kWaves;
  const int groups = (a.n_slots + per_group - 1) / per_group;
  constexpr int rowb = DIM * (FP8 ? 1 : 2);
  constexpr bool stageable = rowb == 128 || rowb == 256;
  const bool staged = stageable && a.cand == nullptr && a.k.page_shift >= 6 && a.k.row_stride == rowb;
  static const int resident_staged =
      resident_workgroups(reinterpret_cast<const void*>(&index_score_mfma<NMT, DIM, FP8, stageable>));
  static const int resident_plain =
      resident_workgroups(reinterpret_cast<const void*>(&index_score_mfma<NMT, DIM, FP8, false>));
  const int gpw = pick_gpw(groups, a.rows.n_rows, staged ? resident_staged : resident_plain);
  dim3 grid((groups + gpw - 1) / gpw, a.rows.n_rows);
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
  const bool chunkable =
      (a.k.block_table == nullptr || (a.k.page_shift >= 6 && a.n_slots <= kPMaxSub * 64)) &&
      a.k.row_stride <= (1 << 24);
  if (fp8 && a.dim == 128 && a.cand == nullptr && a.rows.n_rows >= kPRows && a.n_heads <= 64 && chunkable) {
    const int n_blocks = (a.rows.n_rows + kPRows - 1) / kPRows;
    const int nmt = (a.n_heads + 15) / 16;
    return a.k.block_table ? launch_prefill<true>(a, nmt, n_blocks, s) : launch_prefill<false>(a, nmt, n_blocks, s);
  }
  if (a.dim == 64) return fp8 ? dispatch_heads<64, true>(a, s) : dispatch_heads<64, false>(a, s);
  return fp8 ? dispatch_heads<128, true>(a, s) : dispatch_heads<128, false>(a, s);
}

}  // namespace sa
