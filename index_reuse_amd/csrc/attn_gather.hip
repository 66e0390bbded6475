// Gather attention with one joint softmax over the forced window plus the
// selected entries, on gfx950.
//
// ("HySparse2", section 7.2: window and selected positions come from one KV
// cache and share one softmax normalisation; section 5: the SA layers reuse
// the FA layer's KV and indices with their own queries.  "Lecture 10",
// section 5.1: in MQA mode one latent entry serves every query head, so a
// gathered entry must be shared by all heads to be worth its bytes.)
//
// Work decomposition (BF16 / FP4 KV): one workgroup per (query row, KV head,
// entry split, query-row tile group).  All query heads of the KV group and
// all query sets are stacked into Mq = n_qsets * (Hq / Hkv) MFMA rows, so
// every gathered K/V row is read from HBM once per call and reused by every
// head and query set.  Inside the workgroup, NG entry groups of W waves walk
// disjoint 32-entry tiles of the entry list (several waves per SIMD hide
// each other's latency) and merge their softmax states in LDS at the end.
// Per tile:
//   1. the workgroup gathers the K (and V) rows through the block table
//      into LDS (FP4 rows are dequantised exactly to bf16 on the way);
//   2. each wave computes S^T = K . Q^T for its 16 query rows with
//      v_mfma_f32_16x16x32_bf16 (entries on M, query rows on N), so each lane
//      ends up holding 8 logits of ONE query row;
//   3. softmax in fp32 (exp2 domain) against a per-row reference max fixed
//      by the first tile with a finite logit (a range whose logits outgrow
//      it by 2^64 runs a second time with the true max);
//   4. O^T += V^T . P^T with the contraction order permuted so that the
//      lane's 8 probabilities are directly its B operand; the V^T operand
//      comes straight from LDS through the gfx950 transpose read
//      (ds_read_b64_tr_b16).  O^T keeps each lane on one query
//      row, so the final normalisation needs no cross-lane traffic; row
//      statistics are reduced with the gfx950 lane-swap instructions.
// Long entry lists are split across workgroups; a combine kernel merges the
// (max, sum, unnormalised O) partials.  F32 inputs use a plain VALU kernel.
#include <atomic>
#include <mutex>

#include "kernels.hpp"

namespace sa {

namespace {

constexpr int kTile = 32;   // entries per tile

enum { KV_SEPARATE = 0, KV_SHARED = 1, KV_FP4 = 2 };

// 2^x on the hardware exp unit (v_exp_f32): exact at 0, 0 at -inf; results
// below 2^-126 flush to zero, which softmax weights can afford.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLn2 = 0.6931471805599453f;

// Sink logit of output row (set, head) in log2 units; -inf without a sink.
__device__ __forceinline__ float sink_log2(const AttnArgs& a, int set, int h) {
  return a.sink ? a.sink[set * a.hq + h] * kLog2e : -__builtin_huge_valf();
}

// Final statistics of one output row from its reference m (log2 units), the
// sums l (rounded probabilities, weighting V) and lx (unrounded) relative to
// m, and the sink logit s2 (log2 units, -inf for none): the sink is a virtual
// entry whose value row is zero, so it only adds 2^(s2 - m) to both sums.
// Returns the factor that turns the accumulated O into the output, and the
// natural-log LSE.  Without a sink this is 1 / l and (m + log2 lx) ln 2.
__device__ __forceinline__ float finish_row(float m, float l, float lx, float s2, float& lse) {
  const float M = fmaxf(m, s2);
  if (M == -__builtin_huge_valf()) {
    lse = -__builtin_huge_valf();
    return 0.0f;
  }
  const float f = fast_exp2(m - M), t = fast_exp2(s2 - M);
  const float den = l * f + t, sx = lx * f + t;
  lse = sx > 0.0f ? (M + __log2f(sx)) * kLn2 : -__builtin_huge_valf();
  return den > 0.0f ? f / den : 0.0f;
}

// sigmoid of gate logits: the output gate of each channel
__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + fast_exp2(-x * kLog2e)); }

// Multiply n (4 or 8) consecutive output values of element offset `off` (in
// the o layout) by the sigmoid of their gate logits.
template <int N>
__device__ __forceinline__ void apply_gate(const AttnArgs& a, int64_t off, float (&v)[N]) {
  if (!a.gate) return;
  if (a.dtype == 1) {
    const uint16_t* g = reinterpret_cast<const uint16_t*>(a.gate) + off;
    if constexpr (N == 8) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(g);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] *= sigmoid(__uint_as_float(w[i] << 16));
        v[2 * i + 1] *= sigmoid(__uint_as_float(w[i] & 0xFFFF0000u));
      }
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(g);
      v[0] *= sigmoid(__uint_as_float(w.x << 16));
      v[1] *= sigmoid(__uint_as_float(w.x & 0xFFFF0000u));
      v[2] *= sigmoid(__uint_as_float(w.y << 16));
      v[3] *= sigmoid(__uint_as_float(w.y & 0xFFFF0000u));
    }
  } else {
    const float* g = reinterpret_cast<const float*>(a.gate) + off;
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] *= sigmoid(g[i]);
  }
}

// Store 8 consecutive output channels at element offset `off`.
__device__ __forceinline__ void store8(const AttnArgs& a, int64_t off, const float (&v)[8]) {
  if (a.o_dtype == 1) {
    u32x4 pk;
    pk[0] = pack_bf16x2(v[0], v[1]);
    pk[1] = pack_bf16x2(v[2], v[3]);
    pk[2] = pack_bf16x2(v[4], v[5]);
    pk[3] = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.o) + off) = pk;
  } else {
    float* op = reinterpret_cast<float*>(a.o) + off;
    reinterpret_cast<f32x4*>(op)[0] = f32x4{v[0], v[1], v[2], v[3]};
    reinterpret_cast<f32x4*>(op)[1] = f32x4{v[4], v[5], v[6], v[7]};
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// gfx950 LDS transpose read of 8 bytes (ds_read_b64_tr_b16) at an LDS
// address (8-byte aligned); the lane exchange is described at its use.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}


// Dequantise 32 FP4 channels (16 code bytes, 2 E4M3 scales) into 16 packed
// bf16 pairs.  e2m1 * e4m3 has at most 6 significant bits, so the bf16 value
// is exact and truncating the float is the exact conversion.
__device__ __forceinline__ void fp4_dequant32(u32x4 codes, uint32_t s0, uint32_t s1,
                                              uint32_t out[16]) {
  const float f0 = e4m3_to_f32(s0), f1 = e4m3_to_f32(s1);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t word = codes[w];
    const float sc = w < 2 ? f0 : f1;  // channels 8w..8w+7 -> scale (8w)/16
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t byte = (word >> (8 * p)) & 0xFFu;
      const float lo = e2m1_to_f32(byte & 15u) * sc;
      const float hi = e2m1_to_f32(byte >> 4) * sc;
      out[w * 4 + p] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
    }
  }
}

constexpr int kMaxEntries = 2048;  // entries per workgroup (slot table size)
// Splits per row: attn_combine gives each split one lane of a wave.  The
// entry limit of a call (131072 = 64 x kMaxEntries) never needs more.
constexpr int kMaxSplits = 64;

// Work shape of one workgroup: W waves per entry group, each owning one
// 16-row query tile, and NG entry groups that walk disjoint tiles of the
// entry list (group g takes tiles g, g + NG, ...).  The groups keep their
// own softmax state and merge it in LDS at the end, so several waves per
// SIMD hide each other's LDS and MFMA latency while every gathered row is
// still read from HBM once per workgroup.
template <int DQK, int DV, int KV, int W, int NG, int D>
struct AttnLds {
  static constexpr int KROW = DQK + 8;  // bf16 elements per LDS row (padded)
  static constexpr int VROW = DV + 8;
  static constexpr bool HAS_V = KV == KV_SEPARATE;
  static constexpr int NB = 2 * NG;     // tile buffers: double-buffered per group
  static constexpr int SLOTS = kMaxEntries + (D + 1) * NG * kTile;
  static constexpr int CSTRIDE = 36;    // floats per lane in the merge area
  struct Tiles {
    uint16_t k[NB][kTile * KROW];
    uint16_t v[NB][HAS_V ? kTile * VROW : 1];
  };
  union {
    Tiles t;
    float comb[NG * W * 64 * CSTRIDE];
  } u;
  float ml[NG][W][16][3];  // m, rounded and unrounded probability sums
  int32_t wfirst[W * NG];  // per wave: first entry of the range with a slot
  int32_t slot[SLOTS];     // cache slot of every entry (-1: none)
};

// Per-thread share of one step (NG tiles) of gathered rows, held in
// registers between the global load and the LDS store (the prefetch ring).
template <int DQK, int DV, int KV, int NTH, int NG>
struct TileRegs {
  static constexpr bool FP4 = KV == KV_FP4;
  static constexpr int CPR_K = FP4 ? DQK / 32 : DQK / 8;  // 16-byte chunks per K row
  static constexpr int CPR_V = KV == KV_SEPARATE ? DV / 8 : 0;
  static constexpr int C_K = kTile * CPR_K;
  static constexpr int C_ALL = C_K + kTile * CPR_V;      // chunks per tile
  static constexpr int TOT = NG * C_ALL;                 // chunks per step
  static constexpr int U = (TOT + NTH - 1) / NTH;
  u32x4 v[U];
  uint32_t sc[FP4 ? U : 1];  // FP4: the two E4M3 scales of each 32-channel chunk
};

// ------------------------------------------------------ entry range table
// A workgroup serves entries [e0, e0 + per_split) of its row.
constexpr int kPT = 4;  // table entries per thread per pass

// Range order: the window entries first, then the selected ones, so a row's
// first step can be gathered before its indices are read.  Table entry i
// (entry e = e0 + i) is window position win_lo + e for e < n_w, else the
// selected index idx[e - n_w].  The first pass of index loads assumes n_w
// equals the window parameter (every row with at least that many visible
// entries) and is redone when it does not.
template <int NTH>
__device__ __forceinline__ void issue_index_loads(const AttnArgs& a, int r, int e0, int (&sel_pre)[kPT]) {
  const int32_t* idx = a.idx ? a.idx + (int64_t)r * a.idx_stride : nullptr;
#pragma unroll
  for (int j = 0; j < kPT; ++j)
    sel_pre[j] = idx ? idx[min(max(e0 + j * NTH + (int)threadIdx.x - a.rows.window, 0), a.idx_stride - 1)]
                     : -1;
}

struct RangeTable {
  int ne;          // entries in the range
  int nsteps;      // steps of NG tiles covering them
  int nsteps_run;  // nsteps, or 0 when no entry of the range has a slot
  uint32_t dummy;  // slot read by padding entries
  int n_w;         // window entries of the row
  int n_tab;       // table entries (steps plus the D read ahead)
};

template <int NG, int D>
__device__ __forceinline__ RangeTable range_header(const AttnArgs& a, int r, int e0, int per_split,
                                                   const RowInfo& ri) {
  RangeTable rt;
  rt.n_w = ri.n_avail - ri.win_lo;
  const int cnt = (a.idx && ri.b >= 0) ? a.count[r] : 0;
  const int n_e = ri.b < 0 ? 0 : rt.n_w + cnt;
  const int e1 = min(n_e, e0 + per_split);
  rt.ne = max(0, e1 - e0);
  const int ntiles = (rt.ne + kTile - 1) / kTile;
  rt.nsteps = (ntiles + NG - 1) / NG;
  rt.n_tab = (rt.nsteps + D) * NG * kTile;
  rt.nsteps_run = 0;
  rt.dummy = 0u;
  return rt;
}

// Cache slot of every entry of the range, once, through the block table,
// into slot[] (LDS), entries from `from` on.  Padding to whole steps, and the
// D steps past the end that a prefetch ring reads, are -1.  Loads are
// clamped rather than guarded so that a thread's loads all issue before the
// first wait.  Padding entries later read the rows of the range's first real
// entry: finite data that the mask gives weight exactly 0 (with from > 0 the
// caller has set rt.dummy and rt.nsteps_run already).  `mid` runs once,
// between the issue of the first chunk's block-table reads and their use (a
// caller issues its first gathers there: those reads then go out ahead of
// the gathers and are not held behind them).  Ends with a barrier.
struct NoMid {
  __device__ __forceinline__ void operator()() const {}
};
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

template <int NTH, typename Mid = NoMid>
__device__ __forceinline__ void fill_range_table(const AttnArgs& a, int r, int e0, const RowInfo& ri,
                                                 RangeTable& rt, const int (&sel_pre)[kPT], int from,
                                                 int32_t* slot_tab, int32_t* wfirst_tab,
                                                 Mid mid = Mid()) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* idx = a.idx ? a.idx + (int64_t)r * a.idx_stride : nullptr;
  const bool pre_ok = rt.n_w == a.rows.window;
  int wfirst = 0x7FFFFFFF;
  // selected index of table entry i0 + j NTH + tid (clamped loads)
  auto sel_of = [&](int i0, int (&sel)[kPT]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kPT; ++j)
      sel[j] = idx ? idx[min(max(e0 + i0 + j * NTH + tid - rt.n_w, 0), a.idx_stride - 1)] : -1;
  };
  // One chunk of kPT * NTH table entries.  The block-table case is a
  // compile-time choice and the first chunk is written out apart, so the
  // code from the block-table reads through `hook` to their use has no
  // branch, and the wait for those reads counts exactly the loads `hook`
  // issued after them.
  auto chunk = [&](int i0, const int (&sel)[kPT], auto hook, auto bt) __attribute__((always_inline)) {
    int pos[kPT];
#pragma unroll
    for (int j = 0; j < kPT; ++j) {
      const int i = i0 + j * NTH + tid;
      const int e = e0 + i;
      pos[j] = i < rt.ne ? (e < rt.n_w ? ri.win_lo + e : sel[j]) : -1;
    }
    // block-table reads of the kPT entries, all issued before the first is
    // used (entries without a position read page 0 of the row's table)
    int pg[kPT], off[kPT];
#pragma unroll
    for (int j = 0; j < kPT; ++j) {
      const int e = max(pos[j], 0);
      pg[j] = a.k.page_shift >= 0 ? e >> a.k.page_shift : e / a.k.page_size;
      off[j] = e - pg[j] * a.k.page_size;
    }
    const int64_t row_pages = (int64_t)max(ri.b, 0) * a.k.max_pages;
    int32_t pv[kPT];
    if constexpr (decltype(bt)::value) {
#pragma unroll
      for (int j = 0; j < kPT; ++j) pv[j] = a.k.block_table[row_pages + pg[j]];
    }
    hook();
    // every read is taken here, after all the hook's loads went out (left to
    // itself the compiler sinks a read into the guarded store below, where
    // its wait would cover the hook's loads as well)
    __builtin_amdgcn_sched_barrier(0);
    int64_t page[kPT];
#pragma unroll
    for (int j = 0; j < kPT; ++j) {
      if constexpr (decltype(bt)::value) {
        asm volatile("" ::"v"(pv[j]));
        page[j] = pv[j];
      } else {
        page[j] = row_pages + pg[j];
      }
    }
#pragma unroll
    for (int j = 0; j < kPT; ++j) {
      const int i = i0 + j * NTH + tid;
      const int slot = (ri.b >= 0 && pos[j] >= 0) ? (int)(page[j] * a.k.page_size + off[j]) : -1;
      if (i >= from && i < rt.n_tab) slot_tab[i] = slot;
      // the wave's lowest entry with a slot
      const uint64_t has = __builtin_amdgcn_ballot_w64(slot >= 0);
      if (has) wfirst = min(wfirst, i0 + j * NTH + (tid & ~63) + (int)__builtin_ctzll(has));
    }
  };
  auto run = [&](auto bt) __attribute__((always_inline)) {
    int sel[kPT];
    if (pre_ok) {
#pragma unroll
      for (int j = 0; j < kPT; ++j) sel[j] = sel_pre[j];
    } else {
      sel_of(0, sel);
    }
    chunk(0, sel, mid, bt);
    for (int i0 = kPT * NTH; i0 < rt.n_tab; i0 += kPT * NTH) {
      if (i0 >= rt.ne) {
        // only padding from here on: no index or block-table reads to wait for
#pragma unroll
        for (int j = 0; j < kPT; ++j) {
          const int i = i0 + j * NTH + tid;
          if (i >= from && i < rt.n_tab) slot_tab[i] = -1;
        }
        continue;
      }
      sel_of(i0, sel);
      chunk(i0, sel, NoMid(), bt);
    }
  };
  if (a.k.block_table)
    run(BoolC<true>());
  else
    run(BoolC<false>());
  if (from > 0) {
    __syncthreads();
    return;
  }
  if (lane == 0) wfirst_tab[wave] = wfirst;
  __syncthreads();
  int first = 0x7FFFFFFF;
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) first = min(first, wfirst_tab[w]);
  rt.nsteps_run = first < rt.ne ? rt.nsteps : 0;
  rt.dummy = first < rt.ne ? (uint32_t)slot_tab[first] : 0u;
}

template <int NTH, int NG, int D>
__device__ __forceinline__ RangeTable build_range_table(const AttnArgs& a, int r, int e0, int per_split,
                                                        const RowInfo& ri, const int (&sel_pre)[kPT],
                                                        int32_t* slot_tab, int32_t* wfirst_tab) {
  RangeTable rt = range_header<NG, D>(a, r, e0, per_split, ri);
  fill_range_table<NTH>(a, r, e0, ri, rt, sel_pre, 0, slot_tab, wfirst_tab);
  return rt;
}

// The first n (<= 128) entries of a range that starts with at least that
// many window entries, from scalar block-table reads only (128 consecutive
// entries span at most three pages of 64 or more): their rows can be
// gathered while the indices and their pages are still on the way.  Ends
// with a barrier.
template <int NTH>
__device__ __forceinline__ void fill_window_steps(const AttnArgs& a, const RowInfo& ri, int n,
                                                  int32_t* slot_tab) {
  static_assert(NTH >= 128, "one entry per thread");
  const int pf = ri.win_lo >> a.k.page_shift;
  const int64_t row_pages = (int64_t)ri.b * a.k.max_pages;
  int64_t pgs[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int pk = min(pf + k, a.k.max_pages - 1);
    pgs[k] = a.k.block_table ? (int64_t)a.k.block_table[row_pages + pk] : row_pages + pk;
  }
  const int tid = threadIdx.x;
  if (tid < n) {
    const int pos = ri.win_lo + tid;
    const int k = (pos >> a.k.page_shift) - pf;
    const int64_t page = k == 0 ? pgs[0] : (k == 1 ? pgs[1] : pgs[2]);
    slot_tab[tid] = (int)(page * a.k.page_size + (pos & (a.k.page_size - 1)));
  }
  __syncthreads();
}

// Waves per SIMD that attn_mfma's register budget must leave room for.
// Separate 128-wide rows with a one-step ring fit three (at most 168
// VGPRs), so two 6-wave workgroups share a CU and each hides the other's
// fixed costs and load waits; the others take what they need.
template <int DQK, int KV, int W, int NG, int D>
constexpr int attn_mfma_waves() {
  return (DQK == 128 && KV == KV_SEPARATE && W * NG == 6 && D == 1) ? 3 : 1;
}

template <int DQK, int DV, int KV, int W, int NG, int D>
__global__ __launch_bounds__(64 * W * NG, (attn_mfma_waves<DQK, KV, W, NG, D>())) void attn_mfma(
    AttnArgs a, int per_split) {
  constexpr int NTH = 64 * W * NG;
  using L = AttnLds<DQK, DV, KV, W, NG, D>;
  using T = TileRegs<DQK, DV, KV, NTH, NG>;
  static_assert(sizeof(L) <= 160 * 1024, "LDS budget");
  __shared__ __align__(16) L lds;
  constexpr int KS = DQK / 32;   // k-steps of the S MFMA
  constexpr int QV = DQK / 32;   // 16-byte q vectors per lane
  constexpr int NJB = DV / 128;  // 128-channel blocks of V
  constexpr int NT = DV / 16;    // N tiles of O

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int grp = wave / W, wq = wave - grp * W;
  const int col = lane & 15, gq = lane >> 4;
  const int sp = blockIdx.x;
  const int r = blockIdx.y / a.hkv, g = blockIdx.y % a.hkv;
  const int G = a.hq / a.hkv;
  const int Mq = a.n_qsets * G;
  const int qrow0 = (blockIdx.z * W + wq) * 16;
  const bool active = qrow0 < Mq;

  // The row's first indices, then the query rows of this wave as the B
  // operand (query row = col).  Loads complete in issue order, so the range
  // table, which needs the indices, does not wait for the queries.
  int sel_pre[kPT];
  issue_index_loads<NTH>(a, r, sp * per_split, sel_pre);
  const RowInfo ri = row_info(a.rows, r);  // scalar loads, before any divergent code
  u32x4 qv[QV];
  {
    // unconditional loads (a row past the end reads row 0 and is zeroed), so
    // the wait for the indices below does not have to cover them
    const bool ok = active && qrow0 + col < Mq;
    const int qr = ok ? qrow0 + col : 0;
    const int set = qr / G, h = g * G + qr % G;
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const uint16_t*>(a.q) +
        (((int64_t)set * a.rows.n_rows + r) * a.hq + h) * DQK + gq * (DQK / 4));
#pragma unroll
    for (int i = 0; i < QV; ++i) qv[i] = qp[i];
#pragma unroll
    for (int i = 0; i < QV; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) qv[i][c] = ok ? qv[i][c] : 0u;
  }

  // A range that opens with a whole step of window entries (decode rows
  // with a window) gathers that step while the selected entries' table is
  // built; otherwise the whole table comes first.  (Gathering two window
  // steps early was slower: the larger first burst delays the first data.)
  RangeTable rt = range_header<NG, D>(a, r, sp * per_split, per_split, ri);
  constexpr int SE = NG * kTile;  // entries per step
  static_assert(SE <= 128, "a window step spans at most three pages");
  const bool early =
      sp == 0 && ri.b >= 0 && a.k.page_shift >= 6 && rt.n_w >= SE && rt.ne >= SE;
  if (early) {
    fill_window_steps<NTH>(a, ri, SE, lds.slot);
    rt.dummy = (uint32_t)lds.slot[0];
    rt.nsteps_run = rt.nsteps;
  } else {
    fill_range_table<NTH>(a, r, sp * per_split, ri, rt, sel_pre, 0, lds.slot, lds.wfirst);
  }
  const int ne = rt.ne, nsteps = rt.nsteps, nsteps_run = rt.nsteps_run;
  const uint32_t dummy = rt.dummy;

  // Chunk c of a step: tile c / C_ALL of the step, then K or V row part.
  // Issue the global loads of step s into registers.  Branch-free, so the
  // compiler can keep D steps of loads in flight: an entry without a slot
  // reads slot 0 (always backed by the cache) and is zeroed at store time.
  auto load_step = [&](int s, T& regs) {
#pragma unroll
    for (int u = 0; u < T::U; ++u) {
      int c = tid + NTH * u;
      if (T::TOT % NTH != 0) c = min(c, T::TOT - 1);
      const int gs = c / T::C_ALL;
      const int cw = c - gs * T::C_ALL;
      const bool is_k = cw < T::C_K;
      const int cc = is_k ? cw : cw - T::C_K;
      const int cpr = is_k ? T::CPR_K : T::CPR_V;
      const int e = cc / cpr, part = cc % cpr;
      const int sv = lds.slot[(s * NG + gs) * kTile + e];
      const uint32_t slot = sv >= 0 ? (uint32_t)sv : dummy;
      if constexpr (T::FP4) {
        regs.v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
            a.k.data + (uint64_t)slot * (uint32_t)a.k.row_stride + g * (DQK / 2) + part * 16));
        regs.sc[u] = *reinterpret_cast<const uint16_t*>(
            a.k.scale + (uint64_t)slot * (uint32_t)a.k.scale_stride + g * (DQK / 16) + part * 2);
      } else {
        const char* base =
            is_k ? a.k.data + (uint64_t)slot * (uint32_t)a.k.row_stride + g * (DQK * 2)
                 : a.v.data + (uint64_t)slot * (uint32_t)a.v.row_stride + g * (DV * 2);
        regs.v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + part * 16));
      }
    }
  };
  // Store step s's registers into LDS buffer set `sb` (FP4 is dequantised
  // here).
  auto store_step = [&](const T& regs, int sb) {
#pragma unroll
    for (int u = 0; u < T::U; ++u) {
      const int c = tid + NTH * u;
      if (T::TOT % NTH != 0 && c >= T::TOT) continue;
      const int gs = c / T::C_ALL;
      const int cw = c - gs * T::C_ALL;
      const int buf = sb * NG + gs;
      if constexpr (T::FP4) {
        const int e = cw / T::CPR_K, part = cw % T::CPR_K;
        uint32_t vals[16];
        fp4_dequant32(regs.v[u], regs.sc[u] & 0xFFu, regs.sc[u] >> 8, vals);
        u32x4* dst = reinterpret_cast<u32x4*>(&lds.u.t.k[buf][e * L::KROW + part * 32]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[i] = u32x4{vals[4 * i], vals[4 * i + 1], vals[4 * i + 2], vals[4 * i + 3]};
      } else if (cw < T::C_K) {
        const int e = cw / T::CPR_K, part = cw % T::CPR_K;
        *reinterpret_cast<u32x4*>(&lds.u.t.k[buf][e * L::KROW + part * 8]) = regs.v[u];
      } else {
        const int cc = cw - T::C_K;
        const int e = cc / T::CPR_V, part = cc % T::CPR_V;
        *reinterpret_cast<u32x4*>(&lds.u.t.v[buf][e * L::VROW + part * 8]) = regs.v[u];
      }
    }
  };

  // Softmax state per query row (lane col).  The reference m_run is fixed
  // by the first tile with a finite logit and never moves inside the loop,
  // so O is only ever touched by MFMAs there and stays in accumulation
  // registers.  Probabilities 2^(x - m_run) may exceed 1: they are bf16, so
  // up to 2^kHeadroom they keep full relative precision and O, l stay far
  // from fp32 overflow.  m_top tracks the largest tile max; if it ever
  // exceeds m_run by more than kHeadroom, the range is run a second time with
  // m_run fixed to m_top (every probability then <= 1).
  constexpr float kHeadroom = 64.0f;
  f32x4 O[NT];
  float m_run = -__builtin_huge_valf(), m_top = -__builtin_huge_valf();
  float l_run = 0.0f, l_lse = 0.0f;  // rounded / unrounded probability sums

  // One tile (LDS buffer `buf`, entry tile t) for this wave's query rows.
  auto compute = [&](int buf, int t) {
    const uint16_t* kb = lds.u.t.k[buf];
    // S^T tile: entries (M) x query rows (N)
    f32x4 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = kb + (mt * 16 + col) * L::KROW + gq * (DQK / 4);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 av = *reinterpret_cast<const u32x4*>(krow + ks * 8);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                      __builtin_bit_cast(bf16x8, qv[ks]), acc, 0,
                                                      0, 0);
      }
      s[mt] = acc;
    }
    // mask and scale: lane holds entries mt*16 + 4*gq + i for query row col
    float tmax = -__builtin_huge_valf();
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = mt * 16 + 4 * gq + i;
        const bool ok = lds.slot[t * kTile + e] >= 0;
        const float x = ok ? s[mt][i] * a.scale_log2 : -__builtin_huge_valf();
        s[mt][i] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = xor16_32_max(tmax);
    if (m_run == -__builtin_huge_valf()) m_run = tmax;  // O is still all zero
    m_top = fmaxf(m_top, tmax);
    const float m_use = m_run == -__builtin_huge_valf() ? 0.0f : m_run;
    float p[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[mt][i] = fast_exp2(s[mt][i] - m_use);

    // P^T as the B operand: k-slot 8*gq + i <-> entry (i<4 ? 4gq+i : 16+4gq+i-4)
    u32x4 pa;
    pa[0] = pack_bf16x2(p[0][0], p[0][1]);
    pa[1] = pack_bf16x2(p[0][2], p[0][3]);
    pa[2] = pack_bf16x2(p[1][0], p[1][1]);
    pa[3] = pack_bf16x2(p[1][2], p[1][3]);
    // The output's normaliser sums the same rounded probabilities that weight
    // V, so the output is an exact convex combination of the gathered rows;
    // the log-sum-exp sums the unrounded ones.
    float psum = 0.0f, xsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      psum += __uint_as_float(pa[i] << 16) + __uint_as_float(pa[i] & 0xFFFF0000u);
      xsum += (p[i >> 1][2 * (i & 1)] + p[i >> 1][2 * (i & 1) + 1]);
    }
    l_run += xor16_32_sum(psum);
    l_lse += xor16_32_sum(xsum);
    const bf16x8 pab = __builtin_bit_cast(bf16x8, pa);
    const uint16_t* vbase = KV == KV_SEPARATE ? lds.u.t.v[buf] : kb;
    constexpr int VR = KV == KV_SEPARATE ? L::VROW : L::KROW;
    // V^T as the A operand, straight from LDS with the gfx950 transpose read
    // (ds_read_b64_tr_b16): inside each 16-lane block, lane i receives
    // element i % 4 of the 8 bytes fetched by lanes 4j + i / 4 as its
    // element j.  Lane 4jj + q of k-group gq fetches channels
    // [32q + 4t, 32q + 4t + 4) of entry 4gq + jj (then 16 + 4gq + jj), so
    // lane col gets channel 32(col / 4) + 4t + col % 4 of its k-slots'
    // entries: M-tile 8jb + t row m is channel 128jb + 32(m / 4) + 4t + m % 4.
    const uint16_t* vr0 = vbase + (4 * gq + ((lane >> 2) & 3)) * VR + 32 * (lane & 3);
    const uint16_t* vr1 = vr0 + 16 * VR;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const s16x4 lo = lds_read_tr16(vr0 + jb * 128 + 4 * t);
        const s16x4 hi = lds_read_tr16(vr1 + jb * 128 + 4 * t);
        const s16x8 b = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        O[jb * 8 + t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, b), pab, O[jb * 8 + t], 0, 0, 0);
      }
    }
  };

  // Prefetch ring: step s's rows are loaded D steps ahead of their use.
  // Full groups of D steps run without guards (for even D the LDS buffer set
  // of each unrolled step is static); the last partial group is guarded.
  static_assert(D == 1 || D % 2 == 0, "prefetch depth must be 1 or even");
  T ring[D];
  if (early) {
    // The window step goes out right after the block-table reads of the
    // selected entries (loads complete in issue order, so those reads are
    // not held behind the gathers) and is on its way while the rest of the
    // table is built; the steps after it wait for the table.
    fill_range_table<NTH>(a, r, sp * per_split, ri, rt, sel_pre, SE, lds.slot, lds.wfirst,
                          [&]() { load_step(0, ring[0]); });
  }
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int t = 0; t < NT; ++t) O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < D; ++u)
      if (u > 0 || pass > 0 || !early) load_step(u, ring[u]);
    // One unrolled group of D steps per iteration, the last group guarded
    // step by step (a uniform branch): the tile code appears D times, not 2D
    // (a workgroup with few tiles runs each instruction about once, so code
    // size is instruction-fetch time).  Loads past the last step read the
    // table's D padding steps.
    for (int s0 = 0; s0 < nsteps_run; s0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        if (s0 + u < nsteps_run) {
          const int sb = D % 2 == 0 ? (u & 1) : ((s0 + u) & 1);
          store_step(ring[u], sb);
          // the next loads go out before the barrier: the stores above have
          // read these registers, and the slot table does not change
          load_step(s0 + u + D, ring[u]);
          __syncthreads();
          if (active) compute(sb * NG + grp, (s0 + u) * NG + grp);
        }
      }
    }
    // Every wave of the workgroup takes the same decision (the loop holds
    // barriers); after a second pass m_top == m_run.
    if (!__syncthreads_or(m_top > m_run + kHeadroom)) break;
    m_run = m_top;
    l_run = 0.0f;
    l_lse = 0.0f;
  }

  // Merge the entry groups: every wave publishes (m, l, O^T) in LDS, lane
  // (row, gq) storing its 32 channels as [i][j] (channel 32gq + 8i + j);
  // then wave (grp, wq) finalises channel blocks grp, grp + NG, ... (32
  // channels each) of its 16 query rows over all groups: lane (row, i) sums 8
  // contiguous channels and stores them.
  if constexpr (NG > 1) {
    static_assert(NJB == 1 && 4 % NG == 0, "the group merge spreads 4 channel blocks over the groups");
    __syncthreads();  // every tile buffer is free from here on
    if (gq == 0) {
      lds.ml[grp][wq][col][0] = m_run;
      lds.ml[grp][wq][col][1] = l_run;
      lds.ml[grp][wq][col][2] = l_lse;
    }
    {
      // O[t] holds channels 32gq + 4t + (0..3): the lane's 32 channels in order
      f32x4* dst = reinterpret_cast<f32x4*>(&lds.u.comb[((grp * W + wq) * 64 + lane) * L::CSTRIDE]);
#pragma unroll
      for (int t = 0; t < 8; ++t) dst[t] = O[t];
    }
    __syncthreads();
    if (!active) return;
    const int row = lane & 15, part = lane >> 4;
    const int qr = qrow0 + row;
    if (qr >= Mq) return;
    float M = -__builtin_huge_valf();
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) M = fmaxf(M, lds.ml[gg][wq][row][0]);
    float Ls = 0.0f, Lx = 0.0f, f[NG];
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
      const float m = lds.ml[gg][wq][row][0];
      f[gg] = m == -__builtin_huge_valf() ? 0.0f : fast_exp2(m - M);
      Ls += f[gg] * lds.ml[gg][wq][row][1];
      Lx += f[gg] * lds.ml[gg][wq][row][2];
    }
    const int R = a.rows.n_rows;
    const int set = qr / G, h = g * G + qr % G;
    const int64_t orow = ((int64_t)set * R + r) * a.hq + h;
#pragma unroll
    for (int cb = grp; cb < 4; cb += NG) {
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
      const f32x4* src = reinterpret_cast<const f32x4*>(
          &lds.u.comb[((gg * W + wq) * 64 + row + 16 * cb) * L::CSTRIDE + 8 * part]);
      acc0 += f[gg] * src[0];
      acc1 += f[gg] * src[1];
    }
    const int c0 = 32 * cb + 8 * part;
    if (a.n_split == 1) {
      float lse;
      const float inv = finish_row(M, Ls, Lx, sink_log2(a, set, h), lse);
      float v[8] = {acc0[0] * inv, acc0[1] * inv, acc0[2] * inv, acc0[3] * inv,
                    acc1[0] * inv, acc1[1] * inv, acc1[2] * inv, acc1[3] * inv};
      apply_gate(a, orow * DV + c0, v);
      store8(a, orow * DV + c0, v);
      if (a.lse && cb == 0 && part == 0) a.lse[orow] = lse;
    } else {
      const int64_t nrows = (int64_t)a.n_qsets * R * a.hq;
      float* op = a.part + ((int64_t)sp * nrows + orow) * DV + c0;
      reinterpret_cast<f32x4*>(op)[0] = acc0;
      reinterpret_cast<f32x4*>(op)[1] = acc1;
      if (cb == 0 && part == 0) {
        float* ml = a.part + (int64_t)a.n_split * nrows * DV + ((int64_t)sp * nrows + orow) * 3;
        ml[0] = M;
        ml[1] = Ls;
        ml[2] = Lx;
      }
    }
    }
    return;
  }

  if (!active) return;
  // Output: lane holds O^T for query row qrow0 + col: O[8jb + t][i] is channel
  // 128jb + 32gq + 4t + i, so O[8jb + 2h] and O[8jb + 2h + 1] are the 8
  // contiguous channels from 128jb + 32gq + 8h.
  const int qr = qrow0 + col;
  if (qr >= Mq) return;
  const int R = a.rows.n_rows;
  const int set = qr / G, h = g * G + qr % G;
  const int64_t orow = ((int64_t)set * R + r) * a.hq + h;
  if (a.n_split == 1) {
    float lse;
    const float inv = finish_row(m_run, l_run, l_lse, sink_log2(a, set, h), lse);
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        const int c0 = jb * 128 + 32 * gq + 8 * hh;
        const f32x4 v0 = O[jb * 8 + 2 * hh] * inv, v1 = O[jb * 8 + 2 * hh + 1] * inv;
        float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        apply_gate(a, orow * DV + c0, v);
        store8(a, orow * DV + c0, v);
      }
    if (a.lse && gq == 0) a.lse[orow] = lse;
  } else {
    const int64_t nrows = (int64_t)a.n_qsets * R * a.hq;
    float* po = a.part + ((int64_t)sp * nrows + orow) * DV;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        float* op = po + jb * 128 + 32 * gq + 8 * hh;
        reinterpret_cast<f32x4*>(op)[0] = O[jb * 8 + 2 * hh];
        reinterpret_cast<f32x4*>(op)[1] = O[jb * 8 + 2 * hh + 1];
      }
    if (gq == 0) {
      float* ml = a.part + (int64_t)a.n_split * nrows * DV + ((int64_t)sp * nrows + orow) * 3;
      ml[0] = m_run;
      ml[1] = l_run;
      ml[2] = l_lse;
    }
  }
}

// ------------------------------------------------------- FP4 rows, 4 waves
// FP4 rows (one 512-channel row per entry as K and V, E2M1 codes with E4M3
// scales) with 64 query rows per workgroup (4 waves, one per SIMD; RT = 4
// row tiles of 16).  The rows are decoded to bf16 in registers on their way
// into LDS, so they cannot be loaded straight to LDS as attn_mla_ws does for
// bf16 rows.  Wave w = (hh, dh), hh = w & 1, dh = w >> 1:
//   - S: partial logits of row tiles {2 hh, 2 hh + 1} over k-steps
//     [KH dh, KH dh + KH); every K fragment read from LDS feeds both row
//     tiles;
//   - the two dim halves hand each other the partials of one row tile
//     through LDS; wave w then finishes row tile 2 hh + dh: mask, softmax,
//     and its probabilities (bf16) into LDS;
//   - O: channels [128 w, 128 w + 128) of all four row tiles, so each V
//     channel block is read from LDS by one wave.
// Per 32-entry tile a wave reads 16 KB of K, 8 KB of V and 4 KB of P from
// LDS, against 64 KB of K and V when a wave owns one row tile outright.
// (Two row tiles per workgroup with one K buffer, two workgroups per CU, ran
// 15% slower: each K fragment then feeds one MFMA, with four barriers per
// tile.)
constexpr int kMlaDv = 512, kMlaRT = 4, kMlaD = 1;

template <int DQK>
struct MlaLds {
  static constexpr int RT = kMlaRT, D = kMlaD;
  static constexpr int KROW = DQK + 8;  // bf16 per LDS row (padded)
  static constexpr int SLOTS = kMaxEntries + (D + 1) * kTile;
  uint16_t k[2][kTile * KROW];
  float sx[4][8][64];      // S partials handed to the other dim half
  u32x4 p[RT][64];         // P^T operand of each row tile
  float ml[RT][16][3];     // per row tile: m, rounded and unrounded sums
  int32_t wfirst[4];
  int32_t slot[SLOTS];
};

// The Z query-row groups of one (split, row, KV head) gather the same rows,
// so they run on one XCD at about the same time and the later reads hit that
// XCD's L2: a 1-D grid, workgroups 8 apart in launch order (one XCD) take the
// Z groups of one unit, units rotate over the 8 XCDs.
__device__ __forceinline__ void mla_unit(int n_units, int Z, int& unit, int& z) {
  const int L = blockIdx.x;
  const int rest = L >> 3;
  z = rest % Z;
  unit = (rest / Z) * 8 + (L & 7);
  if (unit >= n_units) unit = -1;
}

// DQK = 512; KV = KV_FP4 (E2M1 codes with E4M3 scales, decoded exactly to
// bf16 on the way into LDS).
template <int DQK, int KV>
__global__ __launch_bounds__(256, 1) void attn_mla(AttnArgs a, int per_split, int n_units, int Z) {
  static_assert(KV == KV_FP4, "bf16 rows take attn_mla_ws");
  constexpr int NTH = 256, DV = kMlaDv, RT = kMlaRT, D = kMlaD;
  constexpr int KH = DQK / 64;      // k-steps per dim half
  constexpr int HT = 2;             // row tiles in this wave's S
  using L = MlaLds<DQK>;
  using T = TileRegs<DQK, DV, KV, NTH, 1>;
  static_assert(sizeof(L) <= 160 * 1024, "LDS budget");
  __shared__ __align__(16) L lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, gq = lane >> 4;
  const int hh = wave & 1, dh = wave >> 1;
  const int own = 2 * hh + dh;  // row tile this wave finishes
  int unit, zg;
  mla_unit(n_units, Z, unit, zg);
  if (unit < 0) return;
  const int sp = unit % a.n_split;
  const int ry = unit / a.n_split;
  const int r = ry / a.hkv, g = ry % a.hkv;
  const int G = a.hq / a.hkv;
  const int Mq = a.n_qsets * G;
  const int qrow0 = zg * 16 * RT;

  // this wave's S row tiles, k-steps [KH dh, KH dh + KH), as B operands
  u32x4 qv[HT][KH];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int qr = qrow0 + 16 * (HT * hh + ht) + col;
    if (qr < Mq) {
      const int set = qr / G, h = g * G + qr % G;
      const u32x4* qp = reinterpret_cast<const u32x4*>(
          reinterpret_cast<const uint16_t*>(a.q) +
          (((int64_t)set * a.rows.n_rows + r) * a.hq + h) * DQK + gq * (DQK / 4));
#pragma unroll
      for (int i = 0; i < KH; ++i) qv[ht][i] = qp[KH * dh + i];
    } else {
#pragma unroll
      for (int i = 0; i < KH; ++i) qv[ht][i] = u32x4{0, 0, 0, 0};
    }
  }
  int sel_pre[kPT];
  issue_index_loads<NTH>(a, r, sp * per_split, sel_pre);
  const RowInfo ri = row_info(a.rows, r);
  const RangeTable rt = build_range_table<NTH, 1, D>(a, r, sp * per_split, per_split, ri, sel_pre,
                                                     lds.slot, lds.wfirst);
  const int nsteps_run = rt.nsteps_run;
  const uint32_t dummy = rt.dummy;

  // step s = tile s: 16-byte pieces of its 32 rows, through registers
  static_assert(T::TOT % NTH == 0, "whole pieces per thread");
  auto load_step = [&](int s, T& regs) {
#pragma unroll
    for (int u = 0; u < T::U; ++u) {
      const int c = tid + NTH * u;
      const int e = c / T::CPR_K, part = c % T::CPR_K;
      const int sv = lds.slot[s * kTile + e];
      const uint32_t slot = sv >= 0 ? (uint32_t)sv : dummy;
      regs.v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          a.k.data + (uint64_t)slot * (uint32_t)a.k.row_stride + g * (DQK / 2) + part * 16));
      regs.sc[u] = *reinterpret_cast<const uint16_t*>(
          a.k.scale + (uint64_t)slot * (uint32_t)a.k.scale_stride + g * (DQK / 16) + part * 2);
    }
  };
  auto store_step = [&](const T& regs, int sb) {
#pragma unroll
    for (int u = 0; u < T::U; ++u) {
      const int c = tid + NTH * u;
      const int e = c / T::CPR_K, part = c % T::CPR_K;
      // 16 code bytes = 32 channels, decoded exactly to bf16
      uint32_t vals[16];
      fp4_dequant32(regs.v[u], regs.sc[u] & 0xFFu, regs.sc[u] >> 8, vals);
      u32x4* dst = reinterpret_cast<u32x4*>(&lds.k[sb][e * L::KROW + part * 32]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dst[i] = u32x4{vals[4 * i], vals[4 * i + 1], vals[4 * i + 2], vals[4 * i + 3]};
    }
  };

  // Softmax state of the finished row tile (lane col), as in attn_mfma: the
  // reference m_run is fixed by the first tile with a finite logit; a
  // second pass runs with m_run = m_top if some tile exceeds it by more than
  // kHeadroom.
  constexpr float kHeadroom = 64.0f;
  f32x4 O[RT][8];  // [row tile][M-tile t]: lane element i is channel 128 w + 32 gq + 4 t + i
  float m_run = -__builtin_huge_valf(), m_top = -__builtin_huge_valf();
  float l_run = 0.0f, l_lse = 0.0f;

  auto compute = [&](int sb, int t) {
    const uint16_t* kb = lds.k[sb];
    // partial S^T tiles [ht][mt]: entries (M) x query rows (N)
    f32x4 s[HT][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 acc[HT];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = kb + (mt * 16 + col) * L::KROW + gq * (DQK / 4) + KH * dh * 8;
#pragma unroll
      for (int i = 0; i < KH; ++i) {
        const u32x4 av = *reinterpret_cast<const u32x4*>(krow + i * 8);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, qv[ht][i]), acc[ht], 0, 0, 0);
      }
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) s[ht][mt] = acc[ht];
    }
    // hand over row tile 1 - dh, take the other half of row tile dh
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) lds.sx[wave][4 * mt + i][lane] = dh ? s[0][mt][i] : s[1][mt][i];
    __syncthreads();
    const int partner = hh + 2 * (1 - dh);
    float x[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        x[mt][i] = (dh ? s[1][mt][i] : s[0][mt][i]) + lds.sx[partner][4 * mt + i][lane];
    // mask and scale: lane holds entries mt*16 + 4*gq + i for query row col
    float tmax = -__builtin_huge_valf();
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = lds.slot[t * kTile + mt * 16 + 4 * gq + i] >= 0;
        x[mt][i] = ok ? x[mt][i] * a.scale_log2 : -__builtin_huge_valf();
        tmax = fmaxf(tmax, x[mt][i]);
      }
    tmax = xor16_32_max(tmax);
    if (m_run == -__builtin_huge_valf()) m_run = tmax;  // O is still all zero
    m_top = fmaxf(m_top, tmax);
    const float m_use = m_run == -__builtin_huge_valf() ? 0.0f : m_run;
    float pr[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[mt][i] = fast_exp2(x[mt][i] - m_use);
    // P^T as the B operand: k-slot 8*gq + i <-> entry (i<4 ? 4gq+i : 16+4gq+i-4)
    u32x4 pa;
    pa[0] = pack_bf16x2(pr[0][0], pr[0][1]);
    pa[1] = pack_bf16x2(pr[0][2], pr[0][3]);
    pa[2] = pack_bf16x2(pr[1][0], pr[1][1]);
    pa[3] = pack_bf16x2(pr[1][2], pr[1][3]);
    float psum = 0.0f, xsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      psum += __uint_as_float(pa[i] << 16) + __uint_as_float(pa[i] & 0xFFFF0000u);
      xsum += pr[i >> 1][2 * (i & 1)] + pr[i >> 1][2 * (i & 1) + 1];
    }
    l_run += xor16_32_sum(psum);
    l_lse += xor16_32_sum(xsum);
    lds.p[own][lane] = pa;
    __syncthreads();
    bf16x8 pb[RT];
#pragma unroll
    for (int q = 0; q < RT; ++q) pb[q] = __builtin_bit_cast(bf16x8, lds.p[q][lane]);
    // V^T as the A operand straight from LDS through the gfx950 transpose
    // read, with attn_mfma's lane layout: M-tile t row m is channel
    // 128 w + 32 (m / 4) + 4 t + m % 4, so accumulator O[q][t][i] of lane
    // (col, gq) holds channel 128 w + 32 gq + 4 t + i of query row col, and
    // the k-slots of each lane are the entries P^T's packing gives them.
    const uint16_t* vr0 = kb + (4 * gq + ((lane >> 2) & 3)) * L::KROW + 32 * (lane & 3) + wave * 128;
    const uint16_t* vr1 = vr0 + 16 * L::KROW;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const s16x4 lo = lds_read_tr16(vr0 + 4 * t);
      const s16x4 hi = lds_read_tr16(vr1 + 4 * t);
      const s16x8 b = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int q = 0; q < RT; ++q)
        O[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b), pb[q],
                                                          O[q][t], 0, 0, 0);
    }
  };

  // One register stage: tile s + 1 loads while tile s is computed from LDS
  // buffer s & 1 (its last readers, tile s - 2, all passed the barrier of
  // tile s - 1).  One loop body keeps every O accumulator in a fixed register
  // (an unrolled pair of bodies made the compiler rotate them between AGPRs).
  static_assert(D == 1, "one register stage");
  T ring;
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int q = 0; q < RT; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) O[q][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    load_step(0, ring);
#pragma unroll 1
    for (int s = 0; s < nsteps_run; ++s) {
      const int sb = s & 1;
      store_step(ring, sb);
      __syncthreads();
      load_step(s + 1, ring);  // past the last tile: the table's padding step
      compute(sb, s);
    }
    if (!__syncthreads_or(m_top > m_run + kHeadroom)) break;
    m_run = m_top;
    l_run = 0.0f;
    l_lse = 0.0f;
  }

  // publish the finished row tile's state, then write channels 128 w.. of
  // all RT row tiles
  if (gq == 0) {
    lds.ml[own][col][0] = m_run;
    lds.ml[own][col][1] = l_run;
    lds.ml[own][col][2] = l_lse;
  }
  __syncthreads();
  const int R_ = a.rows.n_rows;
  if (a.n_split > 1) {
    // Split partials leave through a wave-private transpose in the tile
    // buffers, one row tile at a time (see attn_mla_ws): each store writes
    // two rows' 512-byte runs of the wave's 128 channels.
    constexpr int SROW = 128 + 4;  // floats per staged row
    static_assert(4 * 16 * SROW * 4 <= sizeof(lds.k), "four waves' stages");
    float* stage = reinterpret_cast<float*>(&lds.k[0][0]) + wave * (16 * SROW);
    const int64_t nrows = (int64_t)a.n_qsets * R_ * a.hq;
#pragma unroll
    for (int q = 0; q < RT; ++q) {
      const int qr = qrow0 + 16 * q + col;
      if (qr < Mq && wave == 0 && gq == 0) {
        const int set = qr / G, h = g * G + qr % G;
        const int64_t orow = ((int64_t)set * R_ + r) * a.hq + h;
        float* ml = a.part + (int64_t)a.n_split * nrows * DV + ((int64_t)sp * nrows + orow) * 3;
        ml[0] = lds.ml[q][col][0];
        ml[1] = lds.ml[q][col][1];
        ml[2] = lds.ml[q][col][2];
      }
#pragma unroll
      for (int t = 0; t < 8; ++t)
        *reinterpret_cast<f32x4*>(&stage[col * SROW + 32 * gq + 4 * t]) = O[q][t];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int sr = 2 * k + (lane >> 5);  // staged row: row sr of tile q
        const f32x4 v = *reinterpret_cast<const f32x4*>(&stage[sr * SROW + 4 * (lane & 31)]);
        const int qs = qrow0 + 16 * q + sr;
        if (qs < Mq) {
          const int set = qs / G, h = g * G + qs % G;
          const int64_t orow = ((int64_t)set * R_ + r) * a.hq + h;
          *reinterpret_cast<f32x4*>(a.part + ((int64_t)sp * nrows + orow) * DV + 128 * wave +
                                    4 * (lane & 31)) = v;
        }
      }
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < RT; ++q) {
    const int qr = qrow0 + 16 * q + col;
    if (qr >= Mq) continue;
    const int set = qr / G, h = g * G + qr % G;
    const int64_t orow = ((int64_t)set * R_ + r) * a.hq + h;
    const float m_r = lds.ml[q][col][0], l_r = lds.ml[q][col][1], lx = lds.ml[q][col][2];
    const f32x4* o = O[q];
    if (a.n_split == 1) {
      float lse;
      const float inv = finish_row(m_r, l_r, lx, sink_log2(a, set, h), lse);
#pragma unroll
      for (int hh2 = 0; hh2 < 4; ++hh2) {
        const int c0 = wave * 128 + 32 * gq + 8 * hh2;
        const f32x4 v0 = o[2 * hh2] * inv, v1 = o[2 * hh2 + 1] * inv;
        float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        apply_gate(a, orow * DV + c0, v);
        store8(a, orow * DV + c0, v);
      }
      if (a.lse && wave == 0 && gq == 0) a.lse[orow] = lse;
    } else {
      const int64_t nrows = (int64_t)a.n_qsets * R_ * a.hq;
      float* po = a.part + ((int64_t)sp * nrows + orow) * DV;
#pragma unroll
      for (int hh2 = 0; hh2 < 4; ++hh2) {
        float* op = po + wave * 128 + 32 * gq + 8 * hh2;
        reinterpret_cast<f32x4*>(op)[0] = o[2 * hh2];
        reinterpret_cast<f32x4*>(op)[1] = o[2 * hh2 + 1];
      }
      if (wave == 0 && gq == 0) {
        float* ml = a.part + (int64_t)a.n_split * nrows * DV + ((int64_t)sp * nrows + orow) * 3;
        ml[0] = m_r;
        ml[1] = l_r;
        ml[2] = lx;
      }
    }
  }
}

// ---------------------------------------- load-to-LDS helpers (gfx950)
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// s_waitcnt with only the vector-memory count set (expcnt, lgkmcnt at max).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// Barrier for LDS data only: waits for this wave's LDS operations, not for
// its loads to LDS still in flight (a __syncthreads would wait for those
// too).  The empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------- latent prefill, waves specialised by phase
// The tiling of attn_mla (64 query rows of one KV head per workgroup) for
// bf16 rows: one 576- or 512-wide row per entry, V its first 512 channels,
// on eight waves, two per SIMD, split by role so that the two waves of a
// SIMD are in different phases and one's VALU and LDS work overlaps the
// other's MFMAs:
//   - S waves a = 0..3, (mt, dh) = (a & 1, a >> 1): partial logits of all
//     four row tiles over entry half mt of the 32-entry tile and the k-steps
//     of channel half dh, so every K fragment read from LDS feeds four MFMAs
//     and each tile is read from LDS once; the channel halves swap two row
//     tiles' partials through LDS, and wave a finishes row tiles 2 dh and
//     2 dh + 1 over its entry half: mask, softmax, its half of their P^T
//     operands.  The two entry halves of a row agree on the reference max
//     at tile 0 and add their probability sums at the end.
//   - O waves b = 0..3: channels [128 b, 128 b + 128) of all four row tiles,
//     and every load of the tiles.
// Two barriers per tile.  Before the first, tile s's logits (S waves)
// overlap the reads of tile s - 1's P^T and V (O waves); after it, tile s's
// softmax (S waves) overlaps tile s - 1's O MFMAs, which run from
// registers, and the loads of tile s + 2 into the buffer tile s - 1 has just
// left, which go out among those MFMAs.
// Tiles come from HBM straight into LDS with gfx950's 16-byte load-to-LDS
// (no register staging), two tiles ahead, into three buffers that are
// separate LDS arrays, so the compiler can tell a tile's reads from the
// loads into the other buffers and count the loads still in flight.  Each
// load instruction fills 1 KB of consecutive LDS; rows are laid out 16 bytes
// longer than the data (the lanes that land on a row's pad load the row's
// first piece again), which keeps the MFMA-layout reads of K and the
// transposed reads of V free of bank conflicts.
template <int DQK>
struct MlaWsLds {
  static constexpr int SLOTS = kMaxEntries + 3 * kTile;
  float sx[4][8][64];          // S partials handed to the other channel half
  float sxo[4][8][64];         // at the reference tile: the partials a wave keeps
  u32x4 p[kMlaRT][64];         // P^T operand of each row tile: 8 bytes per entry half
  float mx[4][2][16];          // row max of a wave's two row tiles over its entry half
  float ml[kMlaRT][2][16][3];  // per row tile and entry half: m, rounded and unrounded sums
  int32_t wfirst[8];
  int32_t slot[SLOTS];
};

template <int DQK>
__global__ __launch_bounds__(512, 1) void attn_mla_ws(AttnArgs a, int per_split, int n_units, int Z) {
  constexpr int NTH = 512, DV = kMlaDv, RT = kMlaRT;
  constexpr int P = DQK / 8;                  // 16-byte pieces per row
  constexpr int PP = P + 1;                   // with the pad
  constexpr int KH = DQK / 64;                // k-steps per channel half
  constexpr int JA = (kTile * PP + 255) / 256;  // 1 KB loads per O wave per tile
  constexpr int NJ = 4 * JA;
  using L = MlaWsLds<DQK>;
  static_assert(sizeof(L) + 3 * NJ * 1024 <= 160 * 1024, "LDS budget");
  __shared__ __align__(16) L lds;
  __shared__ __align__(16) u32x4 kb0[NJ * 64];
  __shared__ __align__(16) u32x4 kb1[NJ * 64];
  __shared__ __align__(16) u32x4 kb2[NJ * 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar
  const int col = lane & 15, gq = lane >> 4;
  int unit, zg;
  mla_unit(n_units, Z, unit, zg);
  if (unit < 0) return;
  const int sp = unit % a.n_split;
  const int ry = unit / a.n_split;
  const int r = ry / a.hkv, g = ry % a.hkv;
  const int G = a.hq / a.hkv;
  const int Mq = a.n_qsets * G;
  const int qrow0 = zg * 16 * RT;

  int sel_pre[kPT];
  issue_index_loads<NTH>(a, r, sp * per_split, sel_pre);
  const RowInfo ri = row_info(a.rows, r);
  // two tiles read ahead: the table covers tiles up to nsteps + 1
  const RangeTable rt = build_range_table<NTH, 1, 2>(a, r, sp * per_split, per_split, ri, sel_pre,
                                                     lds.slot, lds.wfirst);
  const int n = rt.nsteps_run;
  constexpr float kHeadroom = 64.0f;

  // The first tile with an entry (n if none; the same in every wave) fixes
  // the reference max of the softmax (see the S waves).
  int s_first = 0;
  while (s_first < n && __builtin_amdgcn_ballot_w64(lds.slot[s_first * kTile + (lane & 31)] >= 0) == 0)
    ++s_first;

  if (wave < 4) {
    // ------------------------------------------------------------ S waves
    // wave (mt, dh): entries [16 mt, 16 mt + 16) of every tile, k-steps
    // [KH dh, KH dh + KH), all four row tiles (every K fragment read from
    // LDS feeds four MFMAs); it finishes row tiles 2 dh and 2 dh + 1 over
    // its entry half
    const int mt = wave & 1, dh = wave >> 1;
    const int partner = wave ^ 2;  // same entries, other channel half
    const int twin = wave ^ 1;     // same row tiles, other entry half
    // qv[j]: row tile (2 dh + j) mod 4, so that j = 0, 1 are the tiles this
    // wave finishes and j = 2, 3 its partner's (static register indices)
    u32x4 qv[RT][KH];
#pragma unroll
    for (int j = 0; j < RT; ++j) {
      const int qr = qrow0 + 16 * ((2 * dh + j) & 3) + col;
      if (qr < Mq) {
        const int set = qr / G, h = g * G + qr % G;
        const u32x4* qp = reinterpret_cast<const u32x4*>(
            reinterpret_cast<const uint16_t*>(a.q) +
            (((int64_t)set * a.rows.n_rows + r) * a.hq + h) * DQK + gq * (DQK / 4));
#pragma unroll
        for (int i = 0; i < KH; ++i) qv[j][i] = qp[KH * dh + i];
      } else {
#pragma unroll
        for (int i = 0; i < KH; ++i) qv[j][i] = u32x4{0, 0, 0, 0};
      }
    }

    // softmax state of row tiles 2 dh + h (lane col) over entry half mt, per
    // lane over its entries; m_run is shared with the twin
    float m_run[2], m_top[2], l_run[2], l_lse[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      m_run[h] = -__builtin_huge_valf();
      m_top[h] = -__builtin_huge_valf();
      l_run[h] = 0.0f;
      l_lse[h] = 0.0f;
    }
    bool m_set = false;

    auto body = [&](int s, const u32x4* cur) __attribute__((always_inline)) {
      // S^T partials [j]: entries 16 mt + (M), query rows of tile
      // (2 dh + j) mod 4 (N)
      f32x4 acc[RT];
#pragma unroll
      for (int j = 0; j < RT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      const u32x4* krow = cur + (16 * mt + col) * PP + gq * (P / 4) + KH * dh;
      // the slot of entry 16 mt + (lane & 15): whether it is real (read here,
      // beside the K reads, rather than after the barrier)
      const int slot_e = lds.slot[s * kTile + 16 * mt + (lane & 15)];
      u32x4 kf[KH];
#pragma unroll
      for (int i = 0; i < KH; ++i) kf[i] = krow[i];
#pragma unroll
      for (int i = 0; i < KH; ++i) {
#pragma unroll
        for (int j = 0; j < RT; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, kf[i]), __builtin_bit_cast(bf16x8, qv[j][i]), acc[j], 0, 0, 0);
      }
      // the slot and five K fragments ahead, then one more read after each
      // fragment's MFMAs (left to itself the scheduler keeps only two reads
      // ahead; all nine at once would not fit the registers)
      __builtin_amdgcn_sched_group_barrier(0x0100, 6, 0);
#pragma unroll
      for (int i = 0; i < KH; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x0008, RT, 0);
        __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);
      }
      // hand the partner the row tiles it finishes
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) lds.sx[wave][4 * h + i][lane] = acc[2 + h][i];
      const bool ref = !m_set && s == s_first;  // the same in every S wave
      if (ref) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) lds.sxo[wave][4 * h + i][lane] = acc[h][i];
      }
      // every logit MFMA before the barrier: after it the O waves' MFMAs run
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();  // (1) the partials
      float x[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[h][i] = acc[h][i] + lds.sx[partner][4 * h + i][lane];
      // keeps the reads out of a branch on the mask
      asm volatile("" : "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[0][2]), "+v"(x[0][3]), "+v"(x[1][0]),
                   "+v"(x[1][1]), "+v"(x[1][2]), "+v"(x[1][3]));
      // which of the half's 16 entries are real: bit e of the ballot over
      // lanes e = lane & 15
      const uint64_t valid = __builtin_amdgcn_ballot_w64(slot_e >= 0);
      const uint32_t vbits = (uint32_t)valid >> (4 * gq);  // bit i: entry 16 mt + 4 gq + i
      // mask and scale: lane holds entries 16 mt + 4 gq + i for query row col
      float tmax[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        tmax[h] = -__builtin_huge_valf();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = (vbits >> i) & 1;
          x[h][i] = ok ? x[h][i] * a.scale_log2 : -__builtin_huge_valf();
          tmax[h] = fmaxf(tmax[h], x[h][i]);
        }
        m_top[h] = fmaxf(m_top[h], tmax[h]);
      }
      if (ref) {
        // this tile fixes the reference: the max of the row over both entry
        // halves, the other half's logits summed from the twin's partials
        // and its partner's
        const uint64_t ovalid =
            __builtin_amdgcn_ballot_w64(lds.slot[s * kTile + 16 * (1 - mt) + (lane & 15)] >= 0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float om = tmax[h];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float y = lds.sxo[twin][4 * h + i][lane] + lds.sx[twin ^ 2][4 * h + i][lane];
            if ((ovalid >> (4 * gq + i)) & 1) om = fmaxf(om, y * a.scale_log2);
          }
          m_run[h] = xor16_32_max(om);
        }
        m_set = true;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float m_use = m_run[h] == -__builtin_huge_valf() ? 0.0f : m_run[h];
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(x[h][i] - m_use);
        // P^T k-slots 8 gq + j: entry 4 gq + j (half 0) in the low 8 bytes,
        // 16 + 4 gq + j (half 1) in the high 8 bytes
        const uint32_t p01 = pack_bf16x2(pr[0], pr[1]), p23 = pack_bf16x2(pr[2], pr[3]);
        // the rounded probabilities' sum (the weights P.V uses), by two
        // bf16 dot products with (1, 1)
        l_run[h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p01), kOnes2, l_run[h],
                                                   false);
        l_run[h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p23), kOnes2, l_run[h],
                                                   false);
        l_lse[h] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
        reinterpret_cast<uint2*>(&lds.p[2 * dh + h][lane])[mt] = uint2{p01, p23};
      }
      lds_barrier();  // (2) P^T of tile s; tile s + 1 has landed
    };

    for (int pass = 0; pass < 2; ++pass) {
      lds_barrier();  // tiles 0 and 1 have landed
      int s = 0;
#pragma unroll 1
      for (; s + 3 <= n; s += 3) {
        body(s, kb0);
        body(s + 1, kb1);
        body(s + 2, kb2);
      }
      if (s < n) body(s, kb0);
      if (s + 1 < n) body(s + 1, kb1);
      if (n > 0) {
        // the O waves' last tile
        lds_barrier();
        lds_barrier();
      }
      float m_row[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        m_row[h] = xor16_32_max(m_top[h]);
        if (gq == 0) lds.mx[wave][h][col] = m_row[h];
      }
      if (!__syncthreads_or(m_top[0] > m_run[0] + kHeadroom || m_top[1] > m_run[1] + kHeadroom))
        break;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        m_run[h] = fmaxf(m_row[h], lds.mx[twin][h][col]);
        l_run[h] = 0.0f;
        l_lse[h] = 0.0f;
      }
      m_set = true;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      l_run[h] = xor16_32_sum(l_run[h]);
      l_lse[h] = xor16_32_sum(l_lse[h]);
      if (gq == 0) {
        lds.ml[2 * dh + h][mt][col][0] = m_run[h];
        lds.ml[2 * dh + h][mt][col][1] = l_run[h];
        lds.ml[2 * dh + h][mt][col][2] = l_lse[h];
      }
    }
    __syncthreads();
    return;
  }

  // -------------------------------------------------------------- O waves
  const int b = wave - 4;
  const uint32_t dummy = rt.dummy;
  const char* kbase = reinterpret_cast<const char*>(a.k.data) + (size_t)g * (DQK * 2);
  const uint32_t rstride = (uint32_t)a.k.row_stride;
  // Tile s into buf: load J = b + 4 j fills LDS pieces f = 64 J + lane,
  // piece f % PP of row f / PP (the pad and the lanes past the last row load
  // a valid piece that nothing reads); every O wave issues JA loads a tile,
  // so one wait count leaves exactly the newest tile in flight.
  int dlin[JA];  // row f / PP in the low 8 bits, byte offset in the row above
#pragma unroll
  for (int j = 0; j < JA; ++j) {
    const int f = 64 * (b + 4 * j) + lane;
    const int ps = f % PP;
    dlin[j] = min(f / PP, kTile - 1) | ((ps < P ? ps : 0) * 16) << 8;
  }
  // The slots of a tile's rows are read ahead (tile_addr); the 64-bit
  // addresses are formed at the issue.
  struct TileAddr {
    uint32_t slot[JA];
  };
  auto tile_addr = [&](int s) __attribute__((always_inline)) {
    TileAddr ta;
    int sv[JA];
#pragma unroll
    for (int j = 0; j < JA; ++j) sv[j] = lds.slot[s * kTile + (dlin[j] & 0xFF)];
#pragma unroll
    for (int j = 0; j < JA; ++j) ta.slot[j] = sv[j] >= 0 ? (uint32_t)sv[j] : dummy;
    return ta;
  };
  auto issue_load = [&](const TileAddr& ta, u32x4* buf, int j) __attribute__((always_inline)) {
    const char* src = kbase + (uint64_t)ta.slot[j] * rstride + (uint32_t)(dlin[j] >> 8);
    __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)(buf + 64 * (b + 4 * j)), 16, 0, 0);
  };
  // wait until only the loads of the last tile issued are in flight (the
  // empty asm keeps the compiler from sinking those loads below the wait)
  auto wait_all_but_last = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(JA));
  };

  f32x4 O[RT][8];  // [row tile][t]: lane element i is channel 128 b + 32 gq + 4 t + i
  // Transpose-read addressing of V (see attn_mfma): lane 4 jj + q of k-group
  // gq fetches channels [128 b + 32 q + 4 t, +4) of entry 4 gq + jj (then
  // 16 + 4 gq + jj).  With rows PP pieces apart, the 16 lanes of a k-group
  // fall on distinct banks, and the eight t differ by an immediate offset.
  const int vq = lane & 3;
  const int voff = (4 * gq + ((lane >> 2) & 3)) * (PP * 8) + 128 * b + 32 * vq;
  // Tile s: O update of tile s - 1 from buf, which then takes tile s + 2
  // (the table ends at tile n + 1: the last pass reloads that one).
  // V fragments of the tile being applied: the first half (t < 4) is read
  // during the previous tile's MFMAs, in place of the half they have just
  // consumed, the second half before the tile's first barrier, so the read
  // phase (where the S waves read K) carries half the transpose reads.
  s16x8 vf[8];
  auto read_v = [&](const u32x4* src, int t0) __attribute__((always_inline)) {
    const uint16_t* kb = reinterpret_cast<const uint16_t*>(src);
#pragma unroll
    for (int t = t0; t < t0 + 4; ++t) {
      const s16x4 lo = lds_read_tr16(kb + voff + 4 * t);
      const s16x4 hi = lds_read_tr16(kb + voff + 4 * t + 16 * PP * 8);
      vf[t] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  auto obody = [&](int s, u32x4* buf, const u32x4* nbuf) __attribute__((always_inline)) {
    const TileAddr ta = tile_addr(min(s + 2, n + 1));
    bf16x8 pb[RT];
#pragma unroll
    for (int q = 0; q < RT; ++q) pb[q] = __builtin_bit_cast(bf16x8, lds.p[q][lane]);
    read_v(buf, 4);  // the second half of tile s - 1's V (the first came earlier)
    lds_barrier();  // (1) every wave is past its reads of buf
    // the MFMAs run between the two barriers, while the S waves do their
    // softmax (the scheduling barriers keep the compiler from moving them
    // across either barrier); the loads go out among them.  (Issuing half
    // of them before the first barrier instead, into the buffer that nothing
    // reads then, made the kernel a fifth slower.)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int q = 0; q < RT; ++q)
        O[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf[t]), pb[q],
                                                          O[q][t], 0, 0, 0);
    }
    if constexpr (DQK != 512) __builtin_amdgcn_sched_barrier(0);
    read_v(nbuf, 0);  // the first half of tile s's V, in place of what just went in
#pragma unroll
    for (int t = 4; t < 8; ++t) {
#pragma unroll
      for (int q = 0; q < RT; ++q)
        O[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf[t]), pb[q],
                                                          O[q][t], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < JA; ++j) issue_load(ta, buf, j);
    // The loads go out among the MFMAs, about one after every three: the
    // load unit takes a 1 KB load in about the time of three, and a burst
    // would hold the wave's MFMAs back.  With 512-wide rows the next tile's
    // V reads are paced among them too (with 576-wide rows that spilled).
    if constexpr (DQK == 512) {
      __builtin_amdgcn_sched_group_barrier(0x0008, 16, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x0100, 2, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x0020, 1, 0);  // load
      }
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x0008, 2, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x0020, 1, 0);  // load
      }
    } else {
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x0008, 3, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x0020, 1, 0);  // load
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // tile s + 1 has landed (tile s + 2 may still be in flight)
    wait_all_but_last();
    lds_barrier();  // (2)
  };
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int q = 0; q < RT; ++q)
#pragma unroll
      for (int t = 0; t < 8; ++t) O[q][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      const TileAddr t0 = tile_addr(0);
#pragma unroll
      for (int j = 0; j < JA; ++j) issue_load(t0, kb0, j);
      const TileAddr t1 = tile_addr(1);
#pragma unroll
      for (int j = 0; j < JA; ++j) issue_load(t1, kb1, j);
    }
    wait_all_but_last();
    lds_barrier();
    if (n > 0) {
      // tile 0: no O update yet; kb2 takes tile 2
      const TileAddr ta = tile_addr(min(2, n + 1));
      lds_barrier();
      read_v(kb0, 0);
#pragma unroll
      for (int j = 0; j < JA; ++j) issue_load(ta, kb2, j);
      wait_all_but_last();
      lds_barrier();
    }
    int s = 1;
#pragma unroll 1
    for (; s + 2 <= n; s += 3) {
      obody(s, kb0, kb1);
      obody(s + 1, kb1, kb2);
      obody(s + 2, kb2, kb0);
    }
    if (s <= n) obody(s, kb0, kb1);
    if (s + 1 <= n) obody(s + 1, kb1, kb2);
    const bool again = __syncthreads_or(false);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // every load to LDS has landed
    if (!again) break;
  }
  __syncthreads();  // the S waves' row statistics

  const int R_ = a.rows.n_rows;
  if (a.n_split > 1) {
    // Split partials (fp32) go out through a wave-private transpose in the
    // tile buffers, which nothing uses any more: each store instruction
    // then writes two rows' 512-byte runs of the wave's 128 channels,
    // instead of 16-byte pieces of 16 rows (every workgroup of a split call
    // writes its partials at about the same time, and the scattered pieces
    // took a third of a short call).  Rows are padded by 16 bytes, so the
    // 16 lanes of a write fall on distinct banks; one wave's LDS accesses
    // run in order, so no barrier is needed.  (The same transpose for the
    // final bf16 rows of an unsplit call made the long prefill calls
    // slower.)
    constexpr int SROW = 128 + 4;  // floats per staged row
    static_assert(2 * 2 * 16 * SROW * 4 <= NJ * 64 * 16, "two waves' stages per tile buffer");
    float* stage = reinterpret_cast<float*>(b < 2 ? kb0 : kb1) + (b & 1) * (2 * 16 * SROW);
    const int64_t nrows = (int64_t)a.n_qsets * R_ * a.hq;
#pragma unroll
    for (int q = 0; q < RT; ++q) {
      // the row statistics of the lane's row of tile q
      const int qr = qrow0 + 16 * q + col;
      if (qr < Mq && b == 0 && gq == 0) {
        const int set = qr / G, h = g * G + qr % G;
        const int64_t orow = ((int64_t)set * R_ + r) * a.hq + h;
        float* ml = a.part + (int64_t)a.n_split * nrows * DV + ((int64_t)sp * nrows + orow) * 3;
        ml[0] = lds.ml[q][0][col][0];
        ml[1] = lds.ml[q][0][col][1] + lds.ml[q][1][col][1];
        ml[2] = lds.ml[q][0][col][2] + lds.ml[q][1][col][2];
      }
    }
#pragma unroll
    for (int pq = 0; pq < RT / 2; ++pq) {
      // row tiles 2 pq and 2 pq + 1: staged row 16 h + col holds channels
      // [128 b, 128 b + 128) of row col of tile 2 pq + h
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 8; ++t)
          *reinterpret_cast<f32x4*>(&stage[(16 * h + col) * SROW + 32 * gq + 4 * t]) = O[2 * pq + h][t];
      // lane l stores 4 channels of staged row 2 k + (l >> 5)
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int sr = 2 * k + (lane >> 5);
        const f32x4 v = *reinterpret_cast<const f32x4*>(&stage[sr * SROW + 4 * (lane & 31)]);
        const int qr = qrow0 + 16 * (2 * pq + (sr >> 4)) + (sr & 15);
        if (qr < Mq) {
          const int set = qr / G, h = g * G + qr % G;
          const int64_t orow = ((int64_t)set * R_ + r) * a.hq + h;
          *reinterpret_cast<f32x4*>(a.part + ((int64_t)sp * nrows + orow) * DV + 128 * b +
                                    4 * (lane & 31)) = v;
        }
      }
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < RT; ++q) {
    const int qr = qrow0 + 16 * q + col;
    if (qr >= Mq) continue;
    const int set = qr / G, h = g * G + qr % G;
    const int64_t orow = ((int64_t)set * R_ + r) * a.hq + h;
    const float m_r = lds.ml[q][0][col][0];
    const float l_r = lds.ml[q][0][col][1] + lds.ml[q][1][col][1];
    const float lx = lds.ml[q][0][col][2] + lds.ml[q][1][col][2];
    const int c0 = b * 128 + 32 * gq;
    // channels c0 + 8 c2 + [0, 8): t = 2 c2 and 2 c2 + 1
    f32x4 o8[4][2];
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2) {
      o8[c2][0] = O[q][2 * c2];
      o8[c2][1] = O[q][2 * c2 + 1];
    }
    if (a.n_split == 1) {
      float lse;
      const float inv = finish_row(m_r, l_r, lx, sink_log2(a, set, h), lse);
#pragma unroll
      for (int c2 = 0; c2 < 4; ++c2) {
        const f32x4 v0 = o8[c2][0] * inv, v1 = o8[c2][1] * inv;
        float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        apply_gate(a, orow * DV + c0 + 8 * c2, v);
        store8(a, orow * DV + c0 + 8 * c2, v);
      }
      if (a.lse && b == 0 && gq == 0) a.lse[orow] = lse;
    } else {
      const int64_t nrows = (int64_t)a.n_qsets * R_ * a.hq;
      float* po = a.part + ((int64_t)sp * nrows + orow) * DV + c0;
#pragma unroll
      for (int c2 = 0; c2 < 4; ++c2) {
        reinterpret_cast<f32x4*>(po + 8 * c2)[0] = o8[c2][0];
        reinterpret_cast<f32x4*>(po + 8 * c2)[1] = o8[c2][1];
      }
      if (b == 0 && gq == 0) {
        float* ml = a.part + (int64_t)a.n_split * nrows * DV + ((int64_t)sp * nrows + orow) * 3;
        ml[0] = m_r;
        ml[1] = l_r;
        ml[2] = lx;
      }
    }
  }
}

// Merge split partials: o = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i,
// lse from the unrounded sums lx_i the same way.  One wave per output row:
// lane i < n_split holds split i's (m, l, lx) and its weight; every lane then
// sums 4 consecutive channels per 256-channel block over the splits with
// 16-byte loads.
template <int KS>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nrows = (int64_t)a.n_qsets * a.rows.n_rows * a.hq;
  if (row >= nrows) return;
  const int DV = a.dv, ns = a.n_split;
  const float* ml = a.part + (int64_t)ns * nrows * DV;
  // KS > 0 (at most KS splits of 512 channels): every partial load is issued
  // before the split weights are known (one memory round trip instead of
  // several).  Splits past ns re-read split 0 and get weight 0.  KS = 0: a
  // loop over the splits for any count and width.
  constexpr int kS = KS > 0 ? KS : 1;
  constexpr bool pre = KS > 0;
  f32x4 v[kS][2];
  if (pre) {
#pragma unroll
    for (int sp = 0; sp < kS; ++sp)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        v[sp][h] = *reinterpret_cast<const f32x4*>(
            a.part + ((int64_t)(sp < ns ? sp : 0) * nrows + row) * DV + 4 * lane + 256 * h);
  }
  // lanes past ns read split 0's statistics (unconditional loads) and drop them
  const int sl = lane < ns ? lane : 0;
  float m = ml[((int64_t)sl * nrows + row) * 3];
  float l = ml[((int64_t)sl * nrows + row) * 3 + 1];
  float lx = ml[((int64_t)sl * nrows + row) * 3 + 2];
  if (lane >= ns) {
    m = -__builtin_huge_valf();
    l = 0.0f;
    lx = 0.0f;
  }
  const float M = wave_max(m);
  const float f = (l > 0.0f && M != -__builtin_huge_valf()) ? exp2f(m - M) : 0.0f;
  const float L = wave_sum(f * l), Lx = wave_sum(f * lx);
  const int set = (int)(row / ((int64_t)a.rows.n_rows * a.hq)), h = (int)(row % a.hq);
  float lse;
  const float inv = finish_row(M, L, Lx, sink_log2(a, set, h), lse);
  auto put = [&](f32x4 acc, int c0) {
    acc *= inv;
    if (a.gate) {
      float v[4] = {acc[0], acc[1], acc[2], acc[3]};
      apply_gate(a, row * DV + c0, v);
      acc = f32x4{v[0], v[1], v[2], v[3]};
    }
    if (a.o_dtype == 1) {
      uint2 pk;
      pk.x = pack_bf16x2(acc[0], acc[1]);
      pk.y = pack_bf16x2(acc[2], acc[3]);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.o) + row * DV + c0) = pk;
    } else {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + row * DV + c0) = acc;
    }
  };
  if (pre) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sp = 0; sp < kS; ++sp) {
        const float fs = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), sp));
        acc += fs * v[sp][h];
      }
      put(acc, 4 * lane + 256 * h);
    }
  }
  for (int c0 = 4 * lane; !pre && c0 < DV; c0 += 256) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int sp = 0; sp < ns; ++sp) {
      const float fs = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), sp));
      const f32x4 w = *reinterpret_cast<const f32x4*>(a.part + ((int64_t)sp * nrows + row) * DV + c0);
      acc += fs * w;
    }
    put(acc, c0);
  }
  if (a.lse && lane == 0) a.lse[row] = lse;
}

// F32 path: one wave per (row, KV head, query set, query head); entries in
// chunks of 64 (one per lane), online softmax, lanes own output channels.
constexpr int kF32MaxD = 256;
__global__ __launch_bounds__(256) void attn_f32(AttnArgs a) {
  __shared__ float qsh[4][kF32MaxD * 4];
  __shared__ float psh[4][64];
  __shared__ int64_t ssh[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
  const int G = a.hq / a.hkv;
  const int qr = blockIdx.y * 4 + wave;
  if (qr >= a.n_qsets * G) return;
  const int set = qr / G, h = g * G + qr % G;
  const int R = a.rows.n_rows;
  const int64_t orow = ((int64_t)set * R + r) * a.hq + h;
  const RowInfo ri = row_info(a.rows, r);
  const int n_w = ri.n_avail - ri.win_lo;
  const int cnt = (a.idx && ri.b >= 0) ? a.count[r] : 0;
  const int n_e = ri.b < 0 ? 0 : n_w + cnt;
  const int32_t* idx = a.idx ? a.idx + (int64_t)r * a.idx_stride : nullptr;
  const float* q = reinterpret_cast<const float*>(a.q) + orow * a.dqk;
  float* qs = qsh[wave];
  for (int c = lane; c < a.dqk; c += 64) qs[c] = q[c];
  float m_run = -__builtin_huge_valf(), l_run = 0.0f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const char* vdata = a.kv_kind == KV_SEPARATE ? a.v.data : a.k.data;
  const int64_t vstride = a.kv_kind == KV_SEPARATE ? a.v.row_stride : a.k.row_stride;
  const int vhead_w = a.kv_kind == KV_SEPARATE ? a.dv : a.dqk;
  for (int cb = 0; cb < n_e; cb += 64) {
    const int i = cb + lane;
    float x = -__builtin_huge_valf();
    int64_t slot = -1;
    if (i < n_e) {
      const int pos = i < n_w ? ri.win_lo + i : idx[i - n_w];
      if (pos >= 0) {
        slot = cache_slot(a.k, ri.b, pos);
        const float* kr = reinterpret_cast<const float*>(a.k.data + slot * a.k.row_stride) + g * a.dqk;
        float d = 0.0f;
        for (int c = 0; c < a.dqk; ++c) d = fmaf(qs[c], kr[c], d);
        x = d * a.scale_log2;
      }
    }
    const float m_new = fmaxf(m_run, wave_max(x));
    float p = 0.0f, alpha = 1.0f;
    if (m_new != -__builtin_huge_valf()) {
      p = exp2f(x - m_new);
      alpha = exp2f(m_run - m_new);
    }
    l_run = l_run * alpha + wave_sum(p);
    m_run = m_new;
    psh[wave][lane] = p;
    ssh[wave][lane] = slot;
    __builtin_amdgcn_wave_barrier();
    const int ne = min(64, n_e - cb);
    for (int k = 0; k < 4; ++k) acc[k] *= alpha;
    for (int e = 0; e < ne; ++e) {
      const int64_t sl = ssh[wave][e];
      if (sl < 0) continue;
      const float pe = psh[wave][e];
      const float* vr = reinterpret_cast<const float*>(vdata + sl * vstride) + g * vhead_w;
      for (int k = 0; k < 4; ++k) {
        const int c = lane + 64 * k;
        if (c < a.dv) acc[k] = fmaf(pe, vr[c], acc[k]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  float lse;
  const float inv = finish_row(m_run, l_run, l_run, sink_log2(a, set, h), lse);
  for (int k = 0; k < 4; ++k) {
    const int c = lane + 64 * k;
    if (c >= a.dv) continue;
    float v = acc[k] * inv;
    if (a.gate) v *= sigmoid(reinterpret_cast<const float*>(a.gate)[orow * a.dv + c]);
    if (a.o_dtype == 1)
      reinterpret_cast<uint16_t*>(a.o)[orow * a.dv + c] = (uint16_t)f32_to_bf16_bits(v);
    else
      reinterpret_cast<float*>(a.o)[orow * a.dv + c] = v;
  }
  if (a.lse && lane == 0) a.lse[orow] = lse;
}

// Waves per entry group (one 16-row query tile each) and entry groups per
// workgroup.  Decode with at most three query tiles per KV head (C2: 6 query
// sets x 8 heads = 48 rows) runs 3 x 4 = 12 waves; other shapes 4 x NG.
struct AttnShape {
  int w, ng;
};

AttnShape attn_shape(const AttnArgs& a) {
  const int tiles = (a.n_qsets * (a.hq / a.hkv) + 15) / 16;
  // at most 3 query tiles of 128-wide rows: 2 groups of 3 waves with two
  // 2-tile steps in flight beat 4 groups with one 4-tile step (a lighter
  // group merge, and a finer pipeline)
  if (a.kv_kind == KV_SEPARATE && a.dqk == 128 && tiles <= 3) return {3, 2};
  if (a.kv_kind == KV_SHARED && a.dqk == 128 && tiles <= 3) return {3, 2};
  if (a.dqk >= 256) return {4, 1};
  return {4, 2};
}

// The merge of split partials: all of a row's partial loads at once when the
// splits of 512 channels fit the registers (up to 16), else a loop.
void launch_combine(const AttnArgs& a, int64_t nrows, hipStream_t s) {
  const dim3 grid((unsigned)((nrows + 3) / 4)), block(256);
  if (a.dv == 512 && a.n_split <= 8)
    hipLaunchKernelGGL(attn_combine<8>, grid, block, 0, s, a);
  else if (a.dv == 512 && a.n_split <= 16)
    hipLaunchKernelGGL(attn_combine<16>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(attn_combine<0>, grid, block, 0, s, a);
}

template <int DQK, int DV, int KV, int W, int NG, int D>
hipError_t launch_mfma_attn(const AttnArgs& a, hipStream_t s) {
  const int G = a.hq / a.hkv;
  const int tiles = (a.n_qsets * G + 15) / 16;
  const int groups = (tiles + W - 1) / W;
  const int per = ((a.max_entries + a.n_split - 1) / a.n_split + kTile - 1) / kTile * kTile;
  dim3 grid(a.n_split, a.rows.n_rows * a.hkv, groups);
  hipLaunchKernelGGL((attn_mfma<DQK, DV, KV, W, NG, D>), grid, dim3(64 * W * NG), 0, s, a, per);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  const int64_t nrows = (int64_t)a.n_qsets * a.rows.n_rows * a.hq;
  launch_combine(a, nrows, s);
  return hipGetLastError();
}

template <int DQK, int KV>
hipError_t launch_mla(const AttnArgs& a, hipStream_t s) {
  const int G = a.hq / a.hkv;
  const int groups = (a.n_qsets * G + 16 * kMlaRT - 1) / (16 * kMlaRT);
  const int per = ((a.max_entries + a.n_split - 1) / a.n_split + kTile - 1) / kTile * kTile;
  const int n_units = a.n_split * a.rows.n_rows * a.hkv;
  const int64_t nwg = (int64_t)(n_units + 7) / 8 * 8 * groups;
  hipLaunchKernelGGL((attn_mla<DQK, KV>), dim3((unsigned)nwg), dim3(256), 0, s, a, per, n_units,
                     groups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  const int64_t nrows = (int64_t)a.n_qsets * a.rows.n_rows * a.hq;
  launch_combine(a, nrows, s);
  return hipGetLastError();
}

template <int DQK>
hipError_t launch_mla_ws(const AttnArgs& a, hipStream_t s) {
  const int G = a.hq / a.hkv;
  const int groups = (a.n_qsets * G + 16 * kMlaRT - 1) / (16 * kMlaRT);
  const int per = ((a.max_entries + a.n_split - 1) / a.n_split + kTile - 1) / kTile * kTile;
  const int n_units = a.n_split * a.rows.n_rows * a.hkv;
  const int64_t nwg = (int64_t)(n_units + 7) / 8 * 8 * groups;
  hipLaunchKernelGGL((attn_mla_ws<DQK>), dim3((unsigned)nwg), dim3(512), 0, s, a, per, n_units, groups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  const int64_t nrows = (int64_t)a.n_qsets * a.rows.n_rows * a.hq;
  launch_combine(a, nrows, s);
  return hipGetLastError();
}

template <int DQK, int DV, int KV, int D>
hipError_t launch_shaped(const AttnArgs& a, hipStream_t s) {
  const AttnShape sh = attn_shape(a);
  if (sh.w == 3 && sh.ng == 2) {
    // separate rows: a one-step ring at two workgroups per CU (1-3% faster
    // than two steps at one workgroup per CU, alone or with steps in flight)
    if constexpr (DQK == 128) return launch_mfma_attn<DQK, DV, KV, 3, 2, KV == KV_SEPARATE ? 1 : D>(a, s);
  } else if (sh.ng == 1) {
    if constexpr (DQK >= 256) return launch_mfma_attn<DQK, DV, KV, 4, 1, D>(a, s);
  } else {
    if constexpr (DQK < 256) return launch_mfma_attn<DQK, DV, KV, 4, 2, D>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Splits per row so that the grid covers the chip about twice; never below
// one 32-entry tile per split.
void attn_plan(AttnArgs& a) {
  a.n_split = 1;
  if (a.dtype == 0) return;
  const int G = a.hq / a.hkv;
  const int tiles = (a.n_qsets * G + 15) / 16;
  const int64_t base = (int64_t)a.rows.n_rows * a.hkv * ((tiles + attn_shape(a).w - 1) / attn_shape(a).w);
  const int max_split = (a.max_entries + kTile - 1) / kTile;
  // enough entry ranges to occupy the chip, each within the slot table
  int ns = (a.max_entries + kMaxEntries - 1) / kMaxEntries;
  // wide value rows make split partials expensive: stop at about 64
  // workgroups, but take at least 4 splits (measured on 8 and 16 rows of 64
  // heads over 512 entries), and up to one split per 1024 entries of a long
  // range (the partials then cost at most a quarter of the rows they
  // replace; one split per 512 entries is 3% faster for a call alone, but
  // its partial traffic costs 30% of the throughput with calls in flight)
  const int cap = a.dv >= 512
                      ? (int)max(max((int64_t)4, (64 + base - 1) / base), (int64_t)a.max_entries / 1024)
                      : max_split;
  while (ns < max_split && ns < cap && ns < kMaxSplits && base * ns < 256) ++ns;
  a.n_split = ns < 1 ? 1 : ns;
}

size_t attn_workspace_bytes(const AttnArgs& a) {
  if (a.n_split <= 1) return 0;
  const int64_t nrows = (int64_t)a.n_qsets * a.rows.n_rows * a.hq;
  return (size_t)a.n_split * nrows * (a.dv + 3) * sizeof(float);
}

hipError_t launch_attn_gather(const AttnArgs& a, hipStream_t s) {
  if (a.rows.n_rows == 0) return hipSuccess;
  if (a.dtype == 0) {
    const int G = a.hq / a.hkv;
    dim3 grid(a.rows.n_rows * a.hkv, (a.n_qsets * G + 3) / 4);
    hipLaunchKernelGGL(attn_f32, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  // Rows of 512 or more channels with at least 64 query rows per KV head:
  // the kernels that split S by channel halves across their waves, so each
  // K fragment read from LDS feeds two MFMAs (attn_mla_ws for bf16 rows,
  // attn_mla for FP4 rows).
  const bool many_rows = a.n_qsets * (a.hq / a.hkv) >= 16 * kMlaRT;
  if (a.kv_kind == KV_SEPARATE) {
    if (a.dqk == 128 && a.dv == 128) return launch_shaped<128, 128, KV_SEPARATE, 2>(a, s);
    if (a.dqk == 256 && a.dv == 256) return launch_shaped<256, 256, KV_SEPARATE, 2>(a, s);
  } else if (a.kv_kind == KV_SHARED) {
    if (a.dqk == 576 && a.dv == 512) {
      if (many_rows) return launch_mla_ws<576>(a, s);
      return launch_shaped<576, 512, KV_SHARED, 2>(a, s);
    }
    if (a.dqk == 512 && a.dv == 512) {
      if (many_rows) return launch_mla_ws<512>(a, s);
      return launch_shaped<512, 512, KV_SHARED, 2>(a, s);
    }
    if (a.dqk == 128 && a.dv == 128) return launch_shaped<128, 128, KV_SHARED, 2>(a, s);
  } else if (a.kv_kind == KV_FP4) {
    if (a.dqk == 512 && a.dv == 512) {
      if (many_rows) return launch_mla<512, KV_FP4>(a, s);
      return launch_shaped<512, 512, KV_FP4, 4>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------ allocation-free variant
// Split partials of sparse_attn_gather_fwd_noalloc live in one static device
// array per GPU, so the call needs no workspace argument and allocates
// nothing.  The host never passes the array's name to a kernel (in host code
// it is only a stand-in): its device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// used.  Calls that overlap in time on one GPU share the array and race.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch`, looked up on first use.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

hipError_t launch_attn_gather_noalloc(AttnArgs a, hipStream_t s) {
  if (a.rows.n_rows == 0) return hipSuccess;
  if (attn_workspace_bytes(a) > kNoAllocScratchBytes) return hipErrorInvalidValue;
  a.part = nullptr;
  if (a.n_split > 1) {
    void* p = nullptr;
    const hipError_t e = scratch_address(&p);
    if (e != hipSuccess) return e;
    a.part = reinterpret_cast<float*>(p);
  }
  return launch_attn_gather(a, s);
}

}  // namespace sa
