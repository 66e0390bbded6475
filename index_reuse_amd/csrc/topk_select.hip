// Window + top-k selection and the block-max candidate pool on gfx950.
//
// Token mode ("HySparse2", section 7.2): the candidates of a row are the
// visible entries outside the forced window; keep the first min(k, n) in the
// order (score desc, index asc).  Pool mode ("CSA, HCA and CSA2", section
// 3.2, Hierarchical Sparse Indexer): every aligned block of `block` entries is
// scored by its maximum over visible members, the first max_blocks blocks in
// (max desc, block asc) order are kept and their members form the pool.
//
// Scores become order-preserving uint32 keys (-0 folded onto +0).  The kept
// set is {key > theta} plus the elements with key == theta up to index jstar,
// where (theta, jstar) is the take-th element of the total order.  Decode
// rows are few and long, so the per-element work is spread over chunks of
// 2048 elements on many workgroups and only a small per-row step is serial:
//   1. hist (chunks x rows): a histogram of the top 12 key bits of every
//      chunk, merged into the row's histogram with global atomics;
//   2. threshold (one workgroup per row): the bin of the take-th key; one
//      light pass over the row counts, per chunk, the keys above that bin and
//      gathers the bin's few keys into LDS; a second 12-bit level and an
//      exact comparison rank give (theta, jstar); per-chunk kept counts give
//      each chunk its output offset;
//   3. emit (chunks x rows): each chunk writes its kept indices ascending at
//      its offset (wave-contiguous segments, ballot ranks).
// The output depends only on the total order, never on thread timing.
#include "kernels.hpp"

namespace sa {

namespace {

// ---------------------------------------------------------------- wave ops
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
// row_ror:1/2/4/8 reduce within 16-lane rows; the lane swaps combine rows
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp<0x121>(v));
  v = max(v, dpp<0x122>(v));
  v = max(v, dpp<0x124>(v));
  v = max(v, dpp<0x128>(v));
  auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(a[0], a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(b[0], b[1]);
}
__device__ __forceinline__ int wave_sum_i32(int x) {
  uint32_t v = (uint32_t)x;
  v += dpp<0x121>(v);
  v += dpp<0x122>(v);
  v += dpp<0x124>(v);
  v += dpp<0x128>(v);
  auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = a[0] + a[1];
  auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (int)(b[0] + b[1]);
}
// inclusive prefix sum over the 64 lanes (a few calls per kernel)
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}
__device__ __forceinline__ uint64_t lanes_below() {
  const int lane = threadIdx.x & 63;
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// ------------------------------------------------------------------ layout
constexpr int kL1Bits = 12;            // level-1 digit: key bits 31..20
constexpr int kL1 = 1 << kL1Bits;      // level-1 bins
constexpr int kL2 = 4096;              // level-2 bins: key bits 19..8
constexpr int kCap1 = 8192;            // LDS slots for the level-1 bin's keys
constexpr int kRankMax = 512;          // largest level-2 bin ranked by comparison
constexpr int kChunk = 2048;           // elements per chunk workgroup
constexpr int kChunkT = 256;           // threads per chunk workgroup
constexpr int kTT = 1024;              // threads of the per-row threshold workgroup
constexpr int kTW = kTT / 64;
constexpr int kMaxChunks = 1024;       // chunks per row (2M elements)
constexpr int kHistStride = kL1 + 64;  // per-row histogram words (+ valid count)
constexpr int kThrWords = 8;           // per-row results: theta, jstar, take, extra

enum { SRC_TOKEN_FULL = 0, SRC_TOKEN_CAND = 1, SRC_BLOCK = 2, SRC_POOL = 3 };

// Float value of an order-preserving key (inverse of order_key).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Workspace views (see topk_workspace_bytes).
struct Ws {
  uint32_t* hist;    // [R][kHistStride], zero on entry, left zero
  uint32_t* thr;     // [R][kThrWords]
  int32_t* offs;     // [R][chunk_stride] output offset of every chunk
  float* beta;       // [R][beta_stride] block maxima (pool mode)
  int64_t chunk_stride;
};

// ----------------------------------------------------------------- sources
// The elements being ranked (KIND fixes how an element's key is formed).
// key() == 0 marks an element that can never be kept: every real score maps
// to a key >= order_key(-inf) > 0.
template <int KIND>
struct Src {
  const float* sc;      // scores (block maxima for SRC_BLOCK)
  const int32_t* list;  // candidate list (SRC_TOKEN_CAND) or pool (SRC_POOL)
  int n;                // elements
  int win_lo;           // kept tokens must lie below this entry

  __device__ __forceinline__ uint32_t key(int j) const {
    if constexpr (KIND == SRC_TOKEN_FULL || KIND == SRC_BLOCK) {
      return order_key(sc[j]);
    } else if constexpr (KIND == SRC_TOKEN_CAND) {
      const int p = list[j];
      return (p >= 0 && p < win_lo) ? order_key(sc[j]) : 0u;
    } else {
      const int p = list[j];
      const bool ok = p >= 0 && p < win_lo;
      return ok ? order_key(sc[ok ? p : 0]) : 0u;
    }
  }
  // key(j) for any j >= 0, with key 0 past the end: the index is clamped so
  // the loads are unconditional (branch-free code keeps them in flight
  // together).  Needs n >= 1.
  __device__ __forceinline__ uint32_t key_c(int j) const {
    const int jc = min(j, n - 1);
    uint32_t k;
    if constexpr (KIND == SRC_TOKEN_FULL || KIND == SRC_BLOCK) {
      k = order_key(sc[jc]);
    } else if constexpr (KIND == SRC_TOKEN_CAND) {
      const int p = list[jc];
      const float x = sc[jc];
      k = (p >= 0 && p < win_lo) ? order_key(x) : 0u;
    } else {
      const int p = list[jc];
      const bool ok = p >= 0 && p < win_lo;
      const float x = sc[ok ? p : 0];
      k = ok ? order_key(x) : 0u;
    }
    return j < n ? k : 0u;
  }
  static constexpr bool may_be_invalid() {
    return KIND == SRC_TOKEN_CAND || KIND == SRC_POOL;
  }
  __device__ __forceinline__ int position(int j) const {
    if constexpr (KIND == SRC_TOKEN_FULL || KIND == SRC_BLOCK) return j;
    else return list[j];
  }
};

template <int KIND>
__device__ __forceinline__ Src<KIND> make_src(const SelectArgs& a, const Ws& ws, int r,
                                              const RowInfo& ri) {
  Src<KIND> s;
  s.win_lo = ri.win_lo;
  s.list = nullptr;
  if constexpr (KIND == SRC_BLOCK) {
    s.sc = ws.beta + (int64_t)r * a.beta_stride;
    s.n = (ri.n_avail + a.block - 1) / a.block;
    s.win_lo = ri.n_avail;
  } else if constexpr (KIND == SRC_POOL) {
    s.sc = a.scores + (int64_t)r * a.score_stride;
    s.list = a.pool + (int64_t)r * a.pool_stride;
    s.n = a.pool_count[r];
  } else if constexpr (KIND == SRC_TOKEN_CAND) {
    s.sc = a.scores + (int64_t)r * a.score_stride;
    s.list = a.cand + (int64_t)r * a.cand_stride;
    s.n = a.cand_count[r];
  } else {
    s.sc = a.scores + (int64_t)r * a.score_stride;
    s.n = ri.win_lo;
  }
  return s;
}

__device__ __forceinline__ bool kept(uint32_t theta, int jstar, uint32_t key, int j) {
  return key != 0u && (key > theta || (key == theta && j <= jstar));
}

// -------------------------------------------------------------- 1. hist
// beta[r][j] = max of the visible scores of block j (one thread per block).
__global__ __launch_bounds__(256) void block_max_kernel(SelectArgs a, Ws ws) {
  const int r = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  const RowInfo ri = row_info(a.rows, r);
  const int nb = (ri.n_avail + a.block - 1) / a.block;
  if (j >= nb) return;
  const float* sc = a.scores + (int64_t)r * a.score_stride;
  const int lo = j * a.block, hi = min(lo + a.block, ri.n_avail);
  float m = sc[lo];
  for (int s = lo + 1; s < hi; ++s) m = fmaxf(m, sc[s]);
  ws.beta[(int64_t)r * a.beta_stride + j] = m;
}

// Level-1 histogram (key bits 31..20) of one chunk, merged into the row's.
template <int KIND>
__global__ __launch_bounds__(kChunkT) void hist_kernel(SelectArgs a, Ws ws) {
  __shared__ uint32_t h[kL1];
  __shared__ uint32_t nvalid;
  const int r = blockIdx.y;
  const RowInfo ri = row_info(a.rows, r);
  const Src<KIND> s = make_src<KIND>(a, ws, r, ri);
  const int j0 = blockIdx.x * kChunk;
  if (j0 >= s.n) return;
  for (int i = threadIdx.x; i < kL1; i += kChunkT) h[i] = 0u;
  if (threadIdx.x == 0) nvalid = 0u;
  __syncthreads();
  int valid = 0;
  uint32_t keys[kChunk / kChunkT];
#pragma unroll
  for (int i = 0; i < kChunk / kChunkT; ++i) keys[i] = s.key_c(j0 + i * kChunkT + (int)threadIdx.x);
#pragma unroll
  for (int i = 0; i < kChunk / kChunkT; ++i) {
    const uint32_t key = keys[i];
    if (key) {
      atomicAdd(&h[key >> (32 - kL1Bits)], 1u);
      ++valid;
    }
  }
  if (Src<KIND>::may_be_invalid()) {
    valid = wave_sum_i32(valid);
    if ((threadIdx.x & 63) == 0) atomicAdd(&nvalid, (uint32_t)valid);
  }
  __syncthreads();
  uint32_t* gh = ws.hist + (int64_t)r * kHistStride;
  for (int i = threadIdx.x; i < kL1; i += kChunkT)
    if (h[i]) atomicAdd(&gh[i], h[i]);
  if (Src<KIND>::may_be_invalid() && threadIdx.x == 0) atomicAdd(&gh[kL1], nvalid);
}

// --------------------------------------------------------- 2. threshold
struct ThrShared {
  uint32_t hist[kL2];
  uint32_t ckey[kCap1];
  int32_t cidx[kCap1];
  int32_t ccnt[kMaxChunks];  // per-chunk counts
  uint32_t wred[kTW];
  uint32_t u[8];
};

// Locate, scanning bins from the top, the bin holding the rank-th (1-based)
// element of a kL2-bin histogram in LDS; writes it and the count above it to
// sh.u[0], sh.u[1].
__device__ __forceinline__ void locate(const uint32_t* hist, int rank, ThrShared& sh) {
  constexpr int BPT = kL2 / kTT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int hi = kL2 - BPT * tid;
  int c[BPT];
  int mine = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    c[q] = (int)hist[hi - 1 - q];
    mine += c[q];
  }
  const int incl = wave_incl_scan(mine);
  if (lane == 63) sh.wred[tid >> 6] = (uint32_t)incl;
  __syncthreads();
  int above = incl - mine;
  for (int w = 0; w < (tid >> 6); ++w) above += (int)sh.wred[w];
  if (above < rank && rank <= above + mine) {
    int acc = above;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      if (acc + c[q] >= rank) {
        sh.u[0] = (uint32_t)(hi - 1 - q);
        sh.u[1] = (uint32_t)acc;
        break;
      }
      acc += c[q];
    }
  }
  __syncthreads();
}

// Per row: (theta, jstar, take) and the output offset of every chunk.
// Element j of the row is visited by thread j % kTT (coalesced loads); its
// chunk is j / kChunk.  Rows longer than kMaxCnt elements keep chunk counts
// in LDS with atomics instead of registers.
template <int KIND, int KPT>
__global__ __launch_bounds__(kTT) void threshold_kernel(SelectArgs a, Ws ws, int kk) {
  __shared__ ThrShared sh;
  const int tid = threadIdx.x, lane = tid & 63;
  const uint64_t below = lanes_below();
  const int r = blockIdx.x;
  const RowInfo ri = row_info(a.rows, r);
  const Src<KIND> s = make_src<KIND>(a, ws, r, ri);
  uint32_t* gh = ws.hist + (int64_t)r * kHistStride;
  uint32_t* thr = ws.thr + (int64_t)r * kThrWords;
  int32_t* offs = ws.offs + (int64_t)r * ws.chunk_stride;
  const int n = s.n;
  const int nch = (n + kChunk - 1) / kChunk;

  for (int i = tid; i < kL1; i += kTT) sh.hist[i] = gh[i];
  const int n_valid = Src<KIND>::may_be_invalid() ? (int)gh[kL1] : n;
  __syncthreads();
  for (int i = tid; i < kHistStride; i += kTT) gh[i] = 0u;  // leave it zero for the next call
  const int take = min(kk, n_valid);

  // How elements are kept: everything valid (mode 1), nothing (mode 0), or
  // by threshold (mode 2).
  int mode = take == 0 ? 0 : (take == n_valid ? 1 : 2);
  uint32_t b1 = 0;
  int need = 0;
  if (mode == 2) {
    locate(sh.hist, take, sh);
    b1 = sh.u[0];
    need = take - (int)sh.u[1];
  }
  const int m1 = mode == 2 ? (int)sh.hist[b1] : 0;
  __syncthreads();

  // One pass: per-chunk counts of certainly-kept (or valid) elements, and the
  // level-1 bin's keys into LDS with a level-2 histogram.
  for (int i = tid; i < nch; i += kTT) sh.ccnt[i] = 0;
  for (int i = tid; i < kL2; i += kTT) sh.hist[i] = 0u;
  if (tid == 0) sh.u[2] = 0u;
  __syncthreads();
  const bool gather = mode == 2 && m1 <= kCap1;
  // Element j = it*kTT*KPT + i*kTT + tid: all KPT loads of a super-chunk are
  // issued before any processing; chunk of slot i is it*KPT/2 + i/2.
  constexpr int CPS = KPT / (kChunk / kTT);  // chunks per super-chunk
  for (int it = 0; it * kTT * KPT < n; ++it) {
    uint32_t kc[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) kc[i] = s.key_c(it * kTT * KPT + i * kTT + tid);
    int cnt[CPS];
#pragma unroll
    for (int q = 0; q < CPS; ++q) cnt[q] = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const uint32_t key = kc[i];
      const uint32_t d1 = key >> 20;
      cnt[i / (kChunk / kTT)] += mode == 1 ? key != 0u : (mode == 2 && key != 0u && d1 > b1);
    }
#pragma unroll
    for (int q = 0; q < CPS; ++q) {
      const int c = it * CPS + q;
      const int v = wave_sum_i32(cnt[q]);
      if (lane == 0 && v && c < nch) atomicAdd(&sh.ccnt[c], v);
    }
    if (gather) {
      // hit bits of this thread's slots, then one wave prefix for the LDS
      // offsets; the (rare) hits are re-read from the cache to be stored
      uint64_t hits = 0;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const uint32_t key = kc[i];
        hits |= (uint64_t)(key != 0u && (key >> 20) == b1) << i;
      }
      const int nh = __popcll(hits);
      const int incl = wave_incl_scan(nh);
      const int wtot = __builtin_amdgcn_readlane(incl, 63);
      uint32_t wbase = 0;
      if (lane == 0 && wtot) wbase = atomicAdd(&sh.u[2], (uint32_t)wtot);
      wbase = __builtin_amdgcn_readlane(wbase, 0);
      uint32_t slot = wbase + (uint32_t)(incl - nh);
      while (hits) {
        const int i = __ffsll((unsigned long long)hits) - 1;
        hits &= hits - 1;
        const int j = it * kTT * KPT + i * kTT + tid;
        const uint32_t key = s.key_c(j);
        sh.ckey[slot] = key;
        sh.cidx[slot] = j;
        atomicAdd(&sh.hist[(key >> 8) & (kL2 - 1)], 1u);
        ++slot;
      }
    }
  }
  __syncthreads();

  uint32_t theta = 0u;
  int jstar = -1;
  if (mode == 2 && gather) {
    locate(sh.hist, need, sh);
    const uint32_t b2 = sh.u[0];
    const int need2 = need - (int)sh.u[1];
    const int m2 = (int)sh.hist[b2];
    const uint32_t pre = (b1 << 20) | (b2 << 8);
    __syncthreads();
    if (m2 <= kRankMax) {
      // compact the level-2 bin, rank it exactly by (key desc, index asc)
      uint32_t* k2 = sh.hist;
      int32_t* j2 = reinterpret_cast<int32_t*>(sh.hist + kRankMax);
      if (tid == 0) sh.u[2] = 0u;
      __syncthreads();
      for (int b0 = 0; b0 < m1; b0 += kTT) {
        const int i = b0 + tid;
        const bool hit = i < m1 && (sh.ckey[i] & 0xFFFFFF00u) == pre;
        const uint64_t mk = __ballot(hit);
        if (mk) {
          const int lead = __ffsll((unsigned long long)mk) - 1;
          uint32_t sl = 0;
          if (lane == lead) sl = atomicAdd(&sh.u[2], (uint32_t)__popcll(mk));
          sl = __builtin_amdgcn_readlane(sl, lead);
          if (hit) {
            const uint32_t slot = sl + (uint32_t)__popcll(mk & below);
            k2[slot] = sh.ckey[i];
            j2[slot] = sh.cidx[i];
          }
        }
      }
      __syncthreads();
      if (tid < m2) {
        const uint32_t ki = k2[tid];
        const int ji = j2[tid];
        int rank = 0;
        for (int l = 0; l < m2; ++l) {
          const uint32_t kl = k2[l];
          rank += kl > ki || (kl == ki && j2[l] < ji);
        }
        if (rank == need2 - 1) {
          sh.u[3] = ki;
          sh.u[4] = (uint32_t)ji;
        }
      }
      __syncthreads();
      theta = sh.u[3];
      jstar = (int)sh.u[4];
      __syncthreads();
    } else {
      // crowded level-2 bin: the last 8 bits by histogram over the LDS keys,
      // then the need3-th tie by index (ties are few relative to the row)
      for (int i = tid; i < 256; i += kTT) sh.hist[i] = 0u;
      __syncthreads();
      for (int i = tid; i < m1; i += kTT)
        if ((sh.ckey[i] & 0xFFFFFF00u) == pre) atomicAdd(&sh.hist[sh.ckey[i] & 255u], 1u);
      __syncthreads();
      if (tid == 0) {
        int above = 0, d = 255;
        for (; d > 0; --d) {
          const int c = (int)sh.hist[d];
          if (above + c >= need2) break;
          above += c;
        }
        sh.u[0] = (uint32_t)d;
        sh.u[1] = (uint32_t)above;
      }
      __syncthreads();
      theta = pre | sh.u[0];
      const int need3 = need2 - (int)sh.u[1];
      // the need3-th smallest index among keys == theta: count, per tie, the
      // ties with a smaller index
      for (int i = tid; i < m1; i += kTT) {
        if (sh.ckey[i] != theta) continue;
        const int ji = sh.cidx[i];
        int rank = 0;
        for (int l = 0; l < m1; ++l) rank += sh.ckey[l] == theta && sh.cidx[l] < ji;
        if (rank == need3 - 1) sh.u[4] = (uint32_t)ji;
      }
      __syncthreads();
      jstar = (int)sh.u[4];
      __syncthreads();
    }
    // chunk counts of the kept keys inside the level-1 bin
    for (int i = tid; i < m1; i += kTT) {
      const int j = sh.cidx[i];
      if (kept(theta, jstar, sh.ckey[i], j)) atomicAdd(&sh.ccnt[j / kChunk], 1);
    }
    __syncthreads();
  } else if (mode == 2) {
    // level-1 bin too crowded for LDS: resolve the remaining 20 key bits by
    // radix passes over the row, then the tie by index, counting kept
    // elements per chunk in the final pass
    uint32_t prefix = b1 << 20, pmask = 0xFFF00000u;
    int remaining = need;
    const int shifts[3] = {12, 4, 0};
    const int widths[3] = {8, 8, 4};
    for (int p = 0; p < 3; ++p) {
      const int shift = shifts[p];
      const uint32_t dmask = (1u << widths[p]) - 1u;
      for (int i = tid; i <= (int)dmask; i += kTT) sh.hist[i] = 0u;
      __syncthreads();
      for (int j = tid; j < n; j += kTT) {
        const uint32_t key = s.key(j);
        if (key != 0u && (key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & dmask], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int above = 0, d = (int)dmask;
        for (; d > 0; --d) {
          const int c = (int)sh.hist[d];
          if (above + c >= remaining) break;
          above += c;
        }
        sh.u[0] = (uint32_t)d;
        sh.u[1] = (uint32_t)above;
      }
      __syncthreads();
      remaining -= (int)sh.u[1];
      prefix |= sh.u[0] << shift;
      pmask |= dmask << shift;
      __syncthreads();
    }
    theta = prefix;
    // ties of theta in index order: per-chunk tie counts, then the chunk
    // holding the remaining-th tie is scanned in order by one wave
    for (int i = tid; i < nch; i += kTT) sh.hist[i] = 0u;
    __syncthreads();
    for (int j = tid; j < n; j += kTT)
      if (s.key(j) == theta) atomicAdd(&sh.hist[j / kChunk], 1u);
    __syncthreads();
    if (tid < 64) {
      int acc = 0, c = 0;
      for (; c < nch; ++c) {
        const int t = (int)sh.hist[c];
        if (acc + t >= remaining) break;
        acc += t;
      }
      // wave 0 walks chunk c in index order
      int found = -1;
      for (int j0 = c * kChunk; j0 < min(n, (c + 1) * kChunk) && found < 0; j0 += 64) {
        const int j = j0 + lane;
        const bool tie = j < n && s.key(j) == theta;
        const uint64_t m = __ballot(tie);
        const int cnt = __popcll(m);
        if (acc + cnt >= remaining) {
          const int want = remaining - acc;  // 1-based within this group
          if (tie && (int)__popcll(m & below) == want - 1) sh.u[4] = (uint32_t)j;
          found = 1;
        }
        acc += cnt;
      }
    }
    __syncthreads();
    jstar = (int)sh.u[4];
    __syncthreads();
    for (int j = tid; j < n; j += kTT) {
      const uint32_t key = s.key(j);
      if ((key >> 20) == b1 && kept(theta, jstar, key, j)) atomicAdd(&sh.ccnt[j / kChunk], 1);
    }
    __syncthreads();
  }

  // exclusive prefix of the chunk counts -> output offsets
  if (tid < 64) {
    int run = 0;
    for (int c0 = 0; c0 < nch; c0 += 64) {
      const int c = c0 + lane;
      const int v = c < nch ? sh.ccnt[c] : 0;
      const int incl = wave_incl_scan(v);
      if (c < nch) offs[c] = run + incl - v;
      run += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  if (tid == 0) {
    thr[0] = mode == 1 ? 0u : (mode == 0 ? 0xFFFFFFFFu : theta);
    thr[1] = (uint32_t)(mode == 1 ? -1 : jstar);
    thr[2] = (uint32_t)take;
  }
}

// ------------------------------------------------------------- 3. emit
// Each chunk writes its kept elements ascending at its offset.  Wave w owns
// the contiguous quarter [w*512, (w+1)*512) of the chunk; lane l holds
// elements q*64 + l, so in-wave order is (q, lane).
template <int KIND>
__global__ __launch_bounds__(kChunkT) void emit_kernel(SelectArgs a, Ws ws, int pool_mode) {
  __shared__ int wtot[kChunkT / 64];
  const int r = blockIdx.y, c = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t below = lanes_below();
  const RowInfo ri = row_info(a.rows, r);
  const Src<KIND> s = make_src<KIND>(a, ws, r, ri);
  const uint32_t* thr = ws.thr + (int64_t)r * kThrWords;
  const uint32_t theta = thr[0];
  const int jstar = (int)thr[1];
  const int take = (int)thr[2];
  const int bs = a.block;
  int32_t* out = pool_mode ? a.pool + (int64_t)r * a.pool_stride : a.idx + (int64_t)r * a.idx_stride;
  if (c == 0) {
    // padding and count (only the last kept block can be partial)
    if (pool_mode) {
      const int nb = s.n;
      int pool_n = take * bs;
      if (take > 0) {
        const uint32_t klast = s.key(nb - 1);
        if (kept(theta, jstar, klast, nb - 1)) pool_n -= nb * bs - ri.n_avail;
      }
      for (int i = pool_n + threadIdx.x; i < a.max_blocks * bs; i += kChunkT) out[i] = -1;
      if (threadIdx.x == 0) a.pool_count[r] = pool_n;
    } else {
      for (int i = take + threadIdx.x; i < a.k; i += kChunkT) out[i] = -1;
      if (threadIdx.x == 0) a.count[r] = take;
    }
  }
  const int j0 = c * kChunk;
  if (take == 0 || j0 >= s.n) return;
  constexpr int Q = kChunk / kChunkT;
  uint32_t keys[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int j = j0 + wave * (kChunk / 4) + q * 64 + lane;
    keys[q] = s.key_c(j);
  }
  uint32_t flags = 0u;
  int tot = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int j = j0 + wave * (kChunk / 4) + q * 64 + lane;
    const bool me = kept(theta, jstar, keys[q], j);
    flags |= (uint32_t)me << q;
    tot += __popcll(__ballot(me));
  }
  if (lane == 0) wtot[wave] = tot;
  __syncthreads();
  int base = ws.offs[(int64_t)r * ws.chunk_stride + c];
  for (int w = 0; w < wave; ++w) base += wtot[w];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const bool me = (flags >> q) & 1u;
    const uint64_t m = __ballot(me);
    if (me) {
      const int j = j0 + wave * (kChunk / 4) + q * 64 + lane;
      const int rank = base + (int)__popcll(m & below);
      if (pool_mode) {
        const int lo = j * bs, mm = min(bs, ri.n_avail - lo);
        for (int u = 0; u < mm; ++u) out[rank * bs + u] = lo + u;
      } else {
        out[rank] = s.position(j);
      }
    }
    base += (int)__popcll(m);
  }
}

template <int KIND>
void run_select(const SelectArgs& a, const Ws& ws, int64_t max_n, int kk, int pool_mode,
                hipStream_t st) {
  const int R = a.rows.n_rows;
  dim3 gc((unsigned)((max_n + kChunk - 1) / kChunk), R);
  hipLaunchKernelGGL(hist_kernel<KIND>, gc, dim3(kChunkT), 0, st, a, ws);
  if (max_n <= kTT * 32)
    hipLaunchKernelGGL((threshold_kernel<KIND, 32>), dim3(R), dim3(kTT), 0, st, a, ws, kk);
  else
    hipLaunchKernelGGL((threshold_kernel<KIND, 64>), dim3(R), dim3(kTT), 0, st, a, ws, kk);
  hipLaunchKernelGGL(emit_kernel<KIND>, gc, dim3(kChunkT), 0, st, a, ws, pool_mode);
}

int64_t chunk_stride(const SelectArgs& a) {
  int64_t n = a.max_elems;
  if (a.pool) n = max(n, a.beta_stride);
  return ((n + kChunk - 1) / kChunk + 15) / 16 * 16;
}

}  // namespace

size_t topk_workspace_bytes(const SelectArgs& a) {
  const int64_t R = a.rows.n_rows;
  size_t b = (size_t)R * (kHistStride + kThrWords) * sizeof(uint32_t);
  b += (size_t)R * chunk_stride(a) * sizeof(int32_t);
  if (a.pool) b += (size_t)R * a.beta_stride * sizeof(float);
  return b;
}

// Workspace: level-1 histograms [R][kHistStride] (zero on entry, left zero),
// per-row thresholds, per-chunk offsets, then (pool mode) block maxima.
hipError_t launch_topk_select(const SelectArgs& a, hipStream_t st) {
  if (a.rows.n_rows == 0) return hipSuccess;
  const int64_t R = a.rows.n_rows;
  Ws ws;
  ws.hist = reinterpret_cast<uint32_t*>(a.beta);
  ws.thr = ws.hist + R * kHistStride;
  ws.chunk_stride = chunk_stride(a);
  ws.offs = reinterpret_cast<int32_t*>(ws.thr + R * kThrWords);
  ws.beta = reinterpret_cast<float*>(ws.offs + R * ws.chunk_stride);
  if ((a.pool ? a.beta_stride : a.max_elems) > (int64_t)kChunk * kMaxChunks) return hipErrorInvalidValue;
  if (a.pool) {
    dim3 g2((unsigned)((a.beta_stride + 255) / 256), a.rows.n_rows);
    hipLaunchKernelGGL(block_max_kernel, g2, dim3(256), 0, st, a, ws);
    run_select<SRC_BLOCK>(a, ws, a.beta_stride, a.max_blocks, 1, st);
  }
  if (a.k > 0) {
    if (a.pool && a.rows.window == 0 && a.max_blocks >= a.k)
      run_select<SRC_POOL>(a, ws, (int64_t)a.max_blocks * a.block, a.k, 0, st);
    else if (a.cand)
      run_select<SRC_TOKEN_CAND>(a, ws, a.cand_stride, a.k, 0, st);
    else
      run_select<SRC_TOKEN_FULL>(a, ws, a.max_elems, a.k, 0, st);
  }
  return hipGetLastError();
}

}  // namespace sa
