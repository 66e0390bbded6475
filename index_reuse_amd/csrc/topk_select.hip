// Window + top-k selection and the block-max candidate pool on gfx950.
//
// Token mode ("HySparse2", section 7.2): the candidates of a row are the
// visible entries outside the forced window; keep the first min(k, n) in the
// order (score desc, index asc).  Pool mode ("CSA, HCA and CSA2", section
// 3.2, Hierarchical Sparse Indexer; "HySparse2", appendix A.1, the first
// generation's selection of 16 blocks of 64 tokens): every aligned block of
// `block` entries is scored by its maximum over its candidates (visible
// entries outside the window), the first max_blocks blocks in (max desc,
// block asc) order are kept and their candidates form the pool.
//
// Scores become order-preserving uint32 keys (-0 folded onto +0; key 0 marks
// a non-candidate).  The kept set is {key > theta} plus the first t elements
// (lowest indices) with key == theta, where theta is the key of the take-th
// element.  Rows are cut into chunks of 2048 elements and every kernel runs
// one workgroup per (chunk, row), so no step of the selection is serial per
// row:
//   1. hist: a histogram of the top 12 key bits of each chunk, merged into
//      the row's histogram with global atomics;
//   2. scan: every chunk derives the threshold bin b1 from the row histogram
//      and records how many of its elements lie above b1; the members of b1
//      (typically a few hundred to a few thousand) are appended to a per-row
//      list with their element index, with the list's min and max key;
//   3. emit: every chunk resolves theta exactly from the member list (two
//      more histogram levels: key bits 19..8, then 7..0), derives its output
//      offset from the chunk counts and the members before it, and writes its
//      kept elements ascending (wave-contiguous segments, ballot ranks).
// Members that all share one key (ties) need no list; a list that overflows
// with distinct keys falls back to scanning the row.  The output depends only
// on the total order, never on thread timing.
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
// inclusive prefix sum over the 64 lanes: row_shr steps inside each 16-lane
// row (lanes shifted in from outside the row read 0), then the row totals
template <int CTRL>
__device__ __forceinline__ int dpp_z(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
  x += dpp_z<0x111>(x);
  x += dpp_z<0x112>(x);
  x += dpp_z<0x114>(x);
  x += dpp_z<0x118>(x);
  const int t0 = __builtin_amdgcn_readlane(x, 15);
  const int t1 = __builtin_amdgcn_readlane(x, 31);
  const int t2 = __builtin_amdgcn_readlane(x, 47);
  x += (lane >= 16 ? t0 : 0) + (lane >= 32 ? t1 : 0) + (lane >= 48 ? t2 : 0);
  return x;
}
__device__ __forceinline__ uint64_t lanes_below() {
  const int lane = threadIdx.x & 63;
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}
// Lanes 0..15 (one DPP row) hold one value per wave of a 16-wave workgroup:
// the row reduces on its own, and lane 0's result is made uniform.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, dpp<0x121>(v));
  v = max(v, dpp<0x122>(v));
  v = max(v, dpp<0x124>(v));
  v = max(v, dpp<0x128>(v));
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ uint32_t row16_min_u32(uint32_t v) {
  return ~row16_max_u32(~v);
}
// inclusive prefix sum inside each 16-lane row
__device__ __forceinline__ int row16_incl_scan(int x) {
  x += dpp_z<0x111>(x);
  x += dpp_z<0x112>(x);
  x += dpp_z<0x114>(x);
  x += dpp_z<0x118>(x);
  return x;
}

// ------------------------------------------------------------------ layout
constexpr int kL1Bits = 12;            // level-1 digit: key bits 31..20
constexpr int kL1 = 1 << kL1Bits;      // level-1 bins
constexpr int kL2 = 4096;              // level-2 bins: key bits 19..8
constexpr int kChunk = 2048;           // elements per chunk workgroup
constexpr int kChunkT = 256;           // threads per chunk workgroup
constexpr int kQ = kChunk / kChunkT;   // elements per thread
constexpr int kCW = kChunkT / 64;      // waves per chunk workgroup
constexpr int kMaxChunks = 1024;       // chunks per row (2M elements)
constexpr int kHistStride = kL1 + 64;  // per-row histogram words (+ valid count)
constexpr int kRecWords = 16;          // per-row record (see Rec)
constexpr int kCapM = 4096;            // member-list capacity per row

enum { SRC_TOKEN_FULL = 0, SRC_TOKEN_CAND = 1, SRC_BLOCK = 2, SRC_POOL = 3 };

// Per-row record words.
enum {
  REC_MCOUNT = 0,  // members of the threshold bin seen (may exceed kCapM)
  REC_MMIN = 1,    // smallest member key
  REC_MMAX = 2,    // largest member key
  REC_B1 = 3,      // threshold bin
  REC_ABOVE = 4,   // elements in bins above it
  REC_TAKE = 5,    // elements to keep
  REC_MODE = 6,    // 0 keep nothing, 1 keep every valid element, 2 threshold
};

// Float value of an order-preserving key (inverse of order_key).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Workspace views (see topk_workspace_bytes).
struct Ws {
  uint32_t* hist;  // [R][kHistStride], cleared by each chunk-path call
  uint32_t* rec;   // [R][kRecWords]
  uint32_t* mkey;  // [R][kCapM] member keys
  int32_t* midx;   // [R][kCapM] member element indices
  int32_t* cgt;    // [R][chunk_stride] elements above the threshold bin, per chunk
  int32_t* cm;     // [R][chunk_stride] members of the threshold bin, per chunk
  float* beta;     // [R][beta_stride] block maxima (pool mode)
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
  // keys of elements j0 + 64 q (q < Q), key 0 past the end.  Every load of
  // a stage is issued before the first one is consumed: left to itself, the
  // scheduler interleaves waits with the issue and keeps only about a dozen
  // loads in flight per wave.  Needs n >= 1.
  template <int Q>
  __device__ __forceinline__ void keys_c(int j0, uint32_t (&k)[Q]) const {
    float x[Q];
    if constexpr (KIND == SRC_TOKEN_FULL || KIND == SRC_BLOCK) {
#pragma unroll
      for (int q = 0; q < Q; ++q) x[q] = sc[min(j0 + 64 * q, n - 1)];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < Q; ++q) k[q] = j0 + 64 * q < n ? order_key(x[q]) : 0u;
    } else if constexpr (KIND == SRC_TOKEN_CAND) {
      int p[Q];
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int jc = min(j0 + 64 * q, n - 1);
        p[q] = list[jc];
        x[q] = sc[jc];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < Q; ++q)
        k[q] = (j0 + 64 * q < n && p[q] >= 0 && p[q] < win_lo) ? order_key(x[q]) : 0u;
    } else {
      int p[Q];
#pragma unroll
      for (int q = 0; q < Q; ++q) p[q] = list[min(j0 + 64 * q, n - 1)];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const bool ok = p[q] >= 0 && p[q] < win_lo;
        x[q] = sc[ok ? p[q] : 0];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < Q; ++q)
        k[q] = (j0 + 64 * q < n && p[q] >= 0 && p[q] < win_lo) ? order_key(x[q]) : 0u;
    }
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
    s.n = (ri.win_lo + a.block - 1) / a.block;  // blocks of the candidates (outside the window)
    s.win_lo = ri.win_lo;
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

// -------------------------------------------------------------- 0. blocks
// beta[r][j] = max of the visible scores of block j (one thread per block).
__global__ __launch_bounds__(256) void block_max_kernel(SelectArgs a, Ws ws) {
  const int r = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  const RowInfo ri = row_info(a.rows, r);
  const int nb = (ri.win_lo + a.block - 1) / a.block;
  if (j >= nb) return;
  const float* sc = a.scores + (int64_t)r * a.score_stride;
  const int lo = j * a.block, hi = min(lo + a.block, ri.win_lo);
  float m;
  if (a.block == 8 && hi - lo == 8 && (reinterpret_cast<uintptr_t>(sc + lo) & 15) == 0) {
    // a whole block of 8 as two 16-byte loads
    const f32x4 u = reinterpret_cast<const f32x4*>(sc + lo)[0];
    const f32x4 v = reinterpret_cast<const f32x4*>(sc + lo)[1];
    m = fmaxf(fmaxf(fmaxf(u[0], u[1]), fmaxf(u[2], u[3])), fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
  } else {
    m = sc[lo];
    for (int s = lo + 1; s < hi; ++s) m = fmaxf(m, sc[s]);
  }
  ws.beta[(int64_t)r * a.beta_stride + j] = m;
}

// Element q of thread t in a chunk: wave-contiguous 512-element segments,
// lane-interleaved inside (coalesced, and in-wave order is (q, lane)).
template <int CHUNK>
__device__ __forceinline__ int chunk_elem(int q) {
  return (threadIdx.x >> 6) * (CHUNK / kCW) + q * 64 + (threadIdx.x & 63);
}

// The bin holding the rank-th (1-based) element counting from the top bin of
// an NB-bin LDS histogram (NB = 256 or 4096); returns (bin, elements in
// higher bins) through u[0], u[1].  Thread t owns bins [NB - BPT(t+1),
// NB - BPT t); every thread of the workgroup takes part.
template <int NB>
__device__ __forceinline__ void locate(const uint32_t* hist, int rank, int* wred, uint32_t* u) {
  constexpr int BPT = NB / kChunkT;
  static_assert(BPT == 1 || BPT % 4 == 0, "bins per thread");
  const int tid = threadIdx.x, lane = tid & 63;
  const int lo = NB - BPT * (tid + 1);
  uint32_t c[BPT];
  if constexpr (BPT == 1) {
    c[0] = hist[lo];
  } else {
#pragma unroll
    for (int v = 0; v < BPT / 4; ++v) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(hist + lo + 4 * v);
      c[4 * v] = x[0];
      c[4 * v + 1] = x[1];
      c[4 * v + 2] = x[2];
      c[4 * v + 3] = x[3];
    }
  }
  int mine = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) mine += (int)c[q];
  const int incl = wave_incl_scan(mine);
  if (lane == 63) wred[tid >> 6] = incl;
  __syncthreads();
  int above = incl - mine;
#pragma unroll
  for (int w = 0; w < kCW - 1; ++w) above += w < (tid >> 6) ? wred[w] : 0;
  if (above < rank && rank <= above + mine) {
    int acc = above;
    int bin = lo, acc_at = above;
    bool found = false;
#pragma unroll
    for (int q = BPT - 1; q >= 0; --q) {  // from this thread's top bin down
      const int cq = (int)c[q];
      if (!found && acc + cq >= rank) {
        bin = lo + q;
        acc_at = acc;
        found = true;
      }
      acc += cq;
    }
    u[0] = (uint32_t)bin;
    u[1] = (uint32_t)acc_at;
  }
  __syncthreads();
}

// Sum over the workgroup (every thread gets it).
__device__ __forceinline__ int block_sum(int v, int* wred) {
  v = wave_sum_i32(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) wred[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
  for (int w = 0; w < kCW; ++w) t += wred[w];
  return t;
}

// ---------------------------------------------------- 0b. clear the counts
// The row histograms (and valid counts) of the call's rows start at zero:
// cleared here by a fill kernel rather than assumed on entry, so a workspace
// carries nothing from one call to the next (any call may share it with any
// other that does not overlap in time, whatever their row counts).
__global__ __launch_bounds__(256) void zero_hist_kernel(Ws ws, int64_t n_vec) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n_vec) reinterpret_cast<u32x4*>(ws.hist)[i] = u32x4{0u, 0u, 0u, 0u};
}

// -------------------------------------------------------------- 1. hist
// Level-1 histogram (key bits 31..20) of one chunk, merged into the row's;
// chunk 0 also resets the row's record for the scan step.
template <int KIND, int CHUNK>
__global__ __launch_bounds__(kChunkT) void hist_kernel(SelectArgs a, Ws ws) {
  __shared__ uint32_t h[kL1];
  __shared__ uint32_t nvalid;
  const int r = blockIdx.y;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    uint32_t* rec = ws.rec + (int64_t)r * kRecWords;
    rec[REC_MCOUNT] = 0u;
    rec[REC_MMIN] = 0xFFFFFFFFu;
    rec[REC_MMAX] = 0u;
  }
  const RowInfo ri = row_info(a.rows, r);
  const Src<KIND> s = make_src<KIND>(a, ws, r, ri);
  const int j0 = blockIdx.x * CHUNK;
  if (j0 >= s.n) return;
  for (int i = threadIdx.x; i < kL1; i += kChunkT) h[i] = 0u;
  if (threadIdx.x == 0) nvalid = 0u;
  __syncthreads();
  int valid = 0;
  uint32_t keys[CHUNK / kChunkT];
#pragma unroll
  for (int q = 0; q < CHUNK / kChunkT; ++q) keys[q] = s.key_c(j0 + chunk_elem<CHUNK>(q));
#pragma unroll
  for (int q = 0; q < CHUNK / kChunkT; ++q) {
    const uint32_t key = keys[q];
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

// -------------------------------------------------------------- 2. scan
template <int KIND, int CHUNK>
__global__ __launch_bounds__(kChunkT) void scan_kernel(SelectArgs a, Ws ws, int kk) {
  __shared__ __align__(16) uint32_t h[kL1];
  __shared__ int wred[kCW];
  __shared__ uint32_t u[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int r = blockIdx.y, c = blockIdx.x;
  const uint32_t* gh = ws.hist + (int64_t)r * kHistStride;
  // the row histogram: 4 x 16 bytes per thread, loaded before anything else
  constexpr int HV = kL1 / 4 / kChunkT;
  u32x4 hv[HV];
#pragma unroll
  for (int v = 0; v < HV; ++v) hv[v] = reinterpret_cast<const u32x4*>(gh)[v * kChunkT + tid];
  const uint32_t gvalid = gh[kL1];
  const RowInfo ri = row_info(a.rows, r);
  const Src<KIND> s = make_src<KIND>(a, ws, r, ri);
  const int n = s.n;
  const int j0 = c * CHUNK;
  if (j0 >= n && c > 0) return;
  // this chunk's keys: issued now, used after the threshold bin is known
  uint32_t keys[CHUNK / kChunkT];
  if (j0 < n) {
#pragma unroll
    for (int q = 0; q < CHUNK / kChunkT; ++q) keys[q] = s.key_c(j0 + chunk_elem<CHUNK>(q));
  }
  uint32_t* rec = ws.rec + (int64_t)r * kRecWords;
#pragma unroll
  for (int v = 0; v < HV; ++v) reinterpret_cast<u32x4*>(h)[v * kChunkT + tid] = hv[v];
  const int n_valid = Src<KIND>::may_be_invalid() ? (int)gvalid : n;
  __syncthreads();
  const int take = min(kk, n_valid);
  const int mode = take == 0 ? 0 : (take == n_valid ? 1 : 2);
  uint32_t b1 = 0;
  int above = 0;
  if (mode == 2) {
    locate<kL1>(h, take, wred, u);
    b1 = u[0];
    above = (int)u[1];
  }
  if (c == 0 && tid == 0) {
    rec[REC_B1] = b1;
    rec[REC_ABOVE] = (uint32_t)above;
    rec[REC_TAKE] = (uint32_t)take;
    rec[REC_MODE] = (uint32_t)mode;
  }
  if (j0 >= n) return;
  int n_gt = 0, n_hit = 0;
  uint32_t hits = 0, kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int q = 0; q < CHUNK / kChunkT; ++q) {
    const uint32_t key = keys[q];
    const uint32_t d = key >> (32 - kL1Bits);
    const bool gt = mode == 1 ? key != 0u : (mode == 2 && d > b1);
    const bool hit = mode == 2 && key != 0u && d == b1;
    n_gt += gt;
    hits |= (uint32_t)hit << q;
    if (hit) {
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    }
  }
  n_hit = __popc(hits);
  const int64_t co = (int64_t)r * ws.chunk_stride + c;
  const int tot_gt = block_sum(n_gt, wred);
  if (mode != 2) {
    if (tid == 0) {
      ws.cgt[co] = tot_gt;
      ws.cm[co] = 0;
    }
    return;
  }
  // append the members: one global atomic per wave
  const int incl = wave_incl_scan(n_hit);
  const int wtot = __builtin_amdgcn_readlane(incl, 63);
  uint32_t wbase = 0;
  if (lane == 0 && wtot) wbase = atomicAdd(&rec[REC_MCOUNT], (uint32_t)wtot);
  wbase = __builtin_amdgcn_readlane(wbase, 0);
  uint32_t slot = wbase + (uint32_t)(incl - n_hit);
  uint32_t* mk = ws.mkey + (int64_t)r * kCapM;
  int32_t* mj = ws.midx + (int64_t)r * kCapM;
#pragma unroll
  for (int q = 0; q < CHUNK / kChunkT; ++q) {
    if ((hits >> q) & 1u) {
      if (slot < (uint32_t)kCapM) {
        mk[slot] = keys[q];
        mj[slot] = j0 + chunk_elem<CHUNK>(q);
      }
      ++slot;
    }
  }
  kmin = ~wave_max_u32(~kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0 && wtot) {
    atomicMin(&rec[REC_MMIN], kmin);
    atomicMax(&rec[REC_MMAX], kmax);
  }
  const int tot_hit = block_sum(n_hit, wred);
  if (tid == 0) {
    ws.cgt[co] = tot_gt;
    ws.cm[co] = tot_hit;
  }
}

// -------------------------------------------------------------- 3. emit
struct __align__(16) EmitShared {
  uint32_t h[kL2];
  uint32_t mk[kCapM];
  int32_t mj[kCapM];
  int wred[kCW];
  int wcnt[kCW][2];
  uint32_t u[4];
};

template <int KIND, int CHUNK>
__global__ __launch_bounds__(kChunkT) void emit_kernel(SelectArgs a, Ws ws, int pool_mode) {
  __shared__ EmitShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = lanes_below();
  const int r = blockIdx.y, c = blockIdx.x;
  const RowInfo ri = row_info(a.rows, r);
  const Src<KIND> s = make_src<KIND>(a, ws, r, ri);
  const int n = s.n;
  const int j0 = c * CHUNK;
  if (j0 >= n && c > 0) return;
  // this chunk's keys: issued first, used at emission
  uint32_t keys[CHUNK / kChunkT];
  if (j0 < n) {
#pragma unroll
    for (int q = 0; q < CHUNK / kChunkT; ++q) keys[q] = s.key_c(j0 + chunk_elem<CHUNK>(q));
  }
  const uint32_t* rec = ws.rec + (int64_t)r * kRecWords;
  const int mode = (int)rec[REC_MODE];
  const int take = (int)rec[REC_TAKE];
  const uint32_t b1 = rec[REC_B1];
  const int above = (int)rec[REC_ABOVE];
  const int m1 = (int)rec[REC_MCOUNT];
  const uint32_t mmin = rec[REC_MMIN], mmax = rec[REC_MMAX];
  const int32_t* cgt = ws.cgt + (int64_t)r * ws.chunk_stride;
  const int32_t* cm = ws.cm + (int64_t)r * ws.chunk_stride;

  // theta, the theta-ties to keep (t_eq) and, for this chunk, the kept
  // elements before it (offset) and the theta-ties before it (e_before)
  uint32_t theta = mode == 1 ? 0u : 0xFFFFFFFFu;
  int t_eq = 0, e_before = 0, e_total = 0, m_gt_before = 0;
  int gt_before = 0;
  for (int i = tid; i < c; i += kChunkT) gt_before += cgt[i];
  gt_before = block_sum(gt_before, sh.wred);
  if (mode == 2) {
    const int need = take - above;
    const uint32_t pre1 = b1 << 20;
    int cnt_gt = above;
    if (mmin == mmax) {
      // every member has the same key: all of them are theta-ties
      theta = mmin;
      int eb = 0;
      for (int i = tid; i < c; i += kChunkT) eb += cm[i];
      e_before = block_sum(eb, sh.wred);
      e_total = m1;
    } else if (m1 <= kCapM) {
      const uint32_t* gmk = ws.mkey + (int64_t)r * kCapM;
      const int32_t* gmj = ws.midx + (int64_t)r * kCapM;
      for (int i = tid; i < kL2; i += kChunkT) sh.h[i] = 0u;
      for (int i0 = 0; i0 < m1; i0 += 4 * kChunkT) {
        uint32_t kv[4];
        int32_t jv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int i = min(i0 + v * kChunkT + tid, m1 - 1);
          kv[v] = gmk[i];
          jv[v] = gmj[i];
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int i = i0 + v * kChunkT + tid;
          if (i < m1) {
            sh.mk[i] = kv[v];
            sh.mj[i] = jv[v];
          }
        }
      }
      __syncthreads();
      for (int i = tid; i < m1; i += kChunkT) atomicAdd(&sh.h[(sh.mk[i] >> 8) & (kL2 - 1)], 1u);
      __syncthreads();
      locate<kL2>(sh.h, need, sh.wred, sh.u);
      const uint32_t b2 = sh.u[0];
      const int above2 = (int)sh.u[1];
      const uint32_t pre2 = pre1 | (b2 << 8);
      __syncthreads();
      for (int i = tid; i < 256; i += kChunkT) sh.h[i] = 0u;
      __syncthreads();
      for (int i = tid; i < m1; i += kChunkT)
        if ((sh.mk[i] & 0xFFFFFF00u) == pre2) atomicAdd(&sh.h[sh.mk[i] & 255u], 1u);
      __syncthreads();
      locate<256>(sh.h, need - above2, sh.wred, sh.u);
      theta = pre2 | sh.u[0];
      cnt_gt = above + above2 + (int)sh.u[1];
      int eb = 0, gb = 0, et = 0;
      for (int i = tid; i < m1; i += kChunkT) {
        const uint32_t k = sh.mk[i];
        const bool before = sh.mj[i] < j0;
        eb += before && k == theta;
        gb += before && k > theta;
        et += k == theta;
      }
      e_before = block_sum(eb, sh.wred);
      m_gt_before = block_sum(gb, sh.wred);
      e_total = block_sum(et, sh.wred);
    } else {
      // the list overflowed with distinct keys: resolve over the whole row
      for (int i = tid; i < kL2; i += kChunkT) sh.h[i] = 0u;
      __syncthreads();
      for (int j = tid; j < n; j += kChunkT) {
        const uint32_t k = s.key(j);
        if (k != 0u && (k >> 20) == b1) atomicAdd(&sh.h[(k >> 8) & (kL2 - 1)], 1u);
      }
      __syncthreads();
      locate<kL2>(sh.h, need, sh.wred, sh.u);
      const uint32_t b2 = sh.u[0];
      const int above2 = (int)sh.u[1];
      const uint32_t pre2 = pre1 | (b2 << 8);
      __syncthreads();
      for (int i = tid; i < 256; i += kChunkT) sh.h[i] = 0u;
      __syncthreads();
      for (int j = tid; j < n; j += kChunkT) {
        const uint32_t k = s.key(j);
        if (k != 0u && (k & 0xFFFFFF00u) == pre2) atomicAdd(&sh.h[k & 255u], 1u);
      }
      __syncthreads();
      locate<256>(sh.h, need - above2, sh.wred, sh.u);
      theta = pre2 | sh.u[0];
      cnt_gt = above + above2 + (int)sh.u[1];
      int eb = 0, gb = 0, et = 0;
      for (int j = tid; j < n; j += kChunkT) {
        const uint32_t k = s.key(j);
        if (k == 0u || (k >> 20) != b1) continue;
        eb += j < j0 && k == theta;
        gb += j < j0 && k > theta;
        et += k == theta;
      }
      e_before = block_sum(eb, sh.wred);
      m_gt_before = block_sum(gb, sh.wred);
      e_total = block_sum(et, sh.wred);
    }
    t_eq = take - cnt_gt;
  }
  const int offset = gt_before + m_gt_before + min(e_before, t_eq);

  // padding and count (only the last block can be partial)
  const int bs = a.block;
  int32_t* out = pool_mode ? a.pool + (int64_t)r * a.pool_stride : a.idx + (int64_t)r * a.idx_stride;
  if (c == 0) {
    if (pool_mode) {
      bool last_kept = false;
      if (mode != 0 && n > 0) {
        const uint32_t kl = s.key(n - 1);
        last_kept = mode == 1 ? kl != 0u : (kl > theta || (kl == theta && e_total - 1 < t_eq));
      }
      const int pool_n = take * bs - (last_kept ? n * bs - ri.win_lo : 0);
      for (int i = pool_n + tid; i < a.max_blocks * bs; i += kChunkT) out[i] = -1;
      if (tid == 0) a.pool_count[r] = pool_n;
    } else {
      for (int i = take + tid; i < a.k; i += kChunkT) out[i] = -1;
      if (tid == 0) a.count[r] = take;
    }
  }
  if (mode == 0 || j0 >= n) return;

  // emission: kept = key > theta, or a theta-tie whose rank among the row's
  // ties (index order) is below t_eq
  int w_gt = 0, w_eq = 0;
#pragma unroll
  for (int q = 0; q < CHUNK / kChunkT; ++q) {
    w_gt += __popcll(__ballot(keys[q] != 0u && keys[q] > theta));
    w_eq += __popcll(__ballot(mode == 2 && keys[q] != 0u && keys[q] == theta));
  }
  if (lane == 0) {
    sh.wcnt[wave][0] = w_gt;
    sh.wcnt[wave][1] = w_eq;
  }
  __syncthreads();
  int o = offset, eseen = e_before;
  for (int w = 0; w < wave; ++w) {
    const int eq = sh.wcnt[w][1];
    o += sh.wcnt[w][0] + max(0, min(eq, t_eq - eseen));
    eseen += eq;
  }
#pragma unroll
  for (int q = 0; q < CHUNK / kChunkT; ++q) {
    const uint32_t k = keys[q];
    const bool gt = k != 0u && k > theta;
    const bool eq = mode == 2 && k != 0u && k == theta;
    const uint64_t me = __ballot(eq);
    const bool keep = gt || (eq && eseen + (int)__popcll(me & below) < t_eq);
    const uint64_t mk = __ballot(keep);
    if (keep) {
      const int j = j0 + chunk_elem<CHUNK>(q);
      const int rank = o + (int)__popcll(mk & below);
      if (pool_mode) {
        const int lo = j * bs, mm = min(bs, ri.win_lo - lo);
        for (int u = 0; u < mm; ++u) out[rank * bs + u] = lo + u;
      } else {
        out[rank] = s.position(j);
      }
    }
    o += (int)__popcll(mk);
    eseen += (int)__popcll(me);
  }
}

// ------------------------------------------------------- one row per workgroup
// For rows of at most kRowT * EPT elements the whole selection runs in one
// workgroup of 1024 threads: the row's keys stay in registers (EPT per
// thread), so the three steps above become one kernel with no global round
// trips between them.
//   - threshold: the histogram range adapts to the keys it still has to
//     split: 4096 bins over [lo, hi] (first the row's min and max valid key,
//     then the threshold bin), so even tightly clustered scores spread over
//     many bins (few LDS atomic collisions) and every pass narrows the range
//     4096-fold: at most three passes reach a single key theta;
//   - emission: wave w owns elements [w * 64 EPT, (w + 1) * 64 EPT), element
//     q of a lane at w * 64 EPT + 64 q + lane (coalesced loads, in-wave order
//     (q, lane)), so ranks come from ballots and one prefix over the waves.
constexpr int kRowT = 1024;           // threads per row workgroup
constexpr int kRowW = kRowT / 64;     // waves per row workgroup
constexpr int kRowBins = 4096;        // histogram bins per pass
constexpr int kRowBpt = kRowBins / kRowT;

constexpr int kRowFew = 64;           // threshold-bin members ranked directly
// Word 3 of a raw buffer resource on CDNA (32-bit dword loads, range-checked
// against the resource's byte size: loads past it return 0).
constexpr int kBufWord3 = 0x00020000;

struct __align__(16) RowShared {
  uint32_t h[kRowBins];
  int wi[kRowW][2];
  uint32_t wu[kRowW][2];
  int wscan[kRowW];
  int wc[kRowW][2];          // per-wave kept counts
  uint32_t u[4];
  uint32_t mkeys[kRowFew];  // 16-byte aligned: read as u32x4
  int rk[kRowFew][2];       // per member: members above it, at least it
  uint32_t mcount;
};
static_assert(offsetof(RowShared, mkeys) % 16 == 0, "aligned member keys");

// The bin holding the rank-th (1-based) element counting from the top bin;
// returns (bin, elements in higher bins, elements in the bin).  Thread t owns
// the kRowBpt bins just below those of thread t - 1, starting from the top,
// and zeroes them once every thread has read its own (ready for the next
// pass).
__device__ __forceinline__ void row_locate(RowShared& sh, int rank, uint32_t& bin, int& above_bin,
                                           int& in_bin) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lo = kRowBins - kRowBpt * (tid + 1);
  const u32x4 c = *reinterpret_cast<const u32x4*>(&sh.h[lo]);
  static_assert(kRowBpt == 4, "four bins per thread");
  const int mine = (int)(c[0] + c[1] + c[2] + c[3]);
  const int incl = wave_incl_scan(mine);
  if (lane == 63) sh.wscan[wave] = incl;
  __syncthreads();
  *reinterpret_cast<u32x4*>(&sh.h[lo]) = u32x4{0u, 0u, 0u, 0u};
  static_assert(kRowW == 16, "one DPP row of wave totals");
  const int wtot = row16_incl_scan(lane < kRowW ? sh.wscan[lane] : 0);
  int above = incl - mine + (wave ? __builtin_amdgcn_readlane(wtot, wave - 1) : 0);
  if (above < rank && rank <= above + mine) {
    int acc = above, b = lo, at = above, cb = 0;
    bool found = false;
#pragma unroll
    for (int q = kRowBpt - 1; q >= 0; --q) {  // from this thread's top bin down
      const int cq = (int)c[q];
      if (!found && acc + cq >= rank) {
        b = lo + q;
        at = acc;
        cb = cq;
        found = true;
      }
      acc += cq;
    }
    sh.u[0] = (uint32_t)b;
    sh.u[1] = (uint32_t)at;
    sh.u[2] = (uint32_t)cb;
  }
  __syncthreads();
  bin = __builtin_amdgcn_readfirstlane(sh.u[0]);
  above_bin = __builtin_amdgcn_readfirstlane((int)sh.u[1]);
  in_bin = __builtin_amdgcn_readfirstlane((int)sh.u[2]);
}

// The row kernel is bound by vector instruction issue (four waves per SIMD),
// so every pass over the keys is kept to a few instructions per key:
//   - scores and block maxima are read with range-checked buffer loads
//     (immediate offsets, no address arithmetic per key);
//   - per-wave counts come from ballots and scalar popcounts;
//   - the threshold key's tie count comes out of the last narrowing step, so
//     the usual case (every tie kept) needs one comparison per key to count
//     and one to emit.
template <int KIND, int EPT>
__global__ __launch_bounds__(kRowT) void row_select_kernel(SelectArgs a, Ws ws, int kk) {
  constexpr bool pool_mode = KIND == SRC_BLOCK;  // blocks expand into the pool
  // every element below n has a valid key
  constexpr bool dense = KIND == SRC_TOKEN_FULL || KIND == SRC_BLOCK;
  __shared__ RowShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = lanes_below();
  const int r = blockIdx.x;
  const RowInfo ri = row_info(a.rows, r);
  const Src<KIND> s = make_src<KIND>(a, ws, r, ri);
  const int n = __builtin_amdgcn_readfirstlane(s.n);
  const int jw = wave * (64 * EPT) + lane;  // element of q = 0
  const int wn = min(max(n - wave * 64 * EPT, 0), 64 * EPT);  // this wave's elements below n
  uint32_t keys[EPT];
  if (n > 0) {
    if constexpr (dense) {
      // Elements jw + 64 q of sixteen consecutive q lie in one 1024-element
      // window; each window gets a resource of its own (base and size are
      // scalar), so one vector offset and immediate offsets address every
      // load, and the range check (vector plus immediate offset against the
      // size) returns 0 past the row.
      float x[EPT];
#pragma unroll
      for (int g = 0; g < (EPT + 15) / 16; ++g) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(s.sc) + 1024 * g, (short)0, max(n - 1024 * g, 0) * (int)sizeof(float),
            kBufWord3);
#pragma unroll
        for (int q = 16 * g; q < min(16 * g + 16, EPT); ++q)
          x[q] = __builtin_bit_cast(float,
                                    __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * jw + 256 * (q & 15), 0, 0));
      }
      if (wn == 64 * EPT) {
#pragma unroll
        for (int q = 0; q < EPT; ++q) keys[q] = order_key(x[q]);
      } else {  // the row ends in this wave: a select per key, no branches
#pragma unroll
        for (int q = 0; q < EPT; ++q) {
          const uint32_t k = order_key(x[q]);
          keys[q] = lane < wn - 64 * q ? k : 0u;
        }
      }
    } else if constexpr (EPT <= 32) {
      s.keys_c(jw, keys);
    } else {  // no registers to spare for a whole stage
#pragma unroll
      for (int q = 0; q < EPT; ++q) keys[q] = s.key_c(jw + 64 * q);
    }
  } else {
#pragma unroll
    for (int q = 0; q < EPT; ++q) keys[q] = 0u;
  }
#pragma unroll
  for (int i = 0; i < kRowBpt; ++i) sh.h[tid + i * kRowT] = 0u;
  if (tid < 2 * kRowFew) (&sh.rk[0][0])[tid] = 0;
  if (tid == 0) sh.mcount = 0u;

  // Valid count, max valid key, and a lower bound on theta: with J =
  // ceil(take / kRowT) <= 2, each thread's J-th largest key (0 if it has
  // fewer) is below J * kRowT >= take keys of the row, so the smallest of
  // them cannot exceed the take-th largest.  Keys under it are never kept
  // and stay out of the histograms.  When every thread holds J valid keys
  // that bound is itself a valid key, so the row's smallest key is not
  // needed.
  const int J = (min(kk, kRowT * EPT) + kRowT - 1) / kRowT;  // the bound is used for J <= 2
  uint32_t kmax = 0u, k2 = 0u;  // this thread's largest and second largest key
  if (J == 2) {
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      k2 = max(k2, min(kmax, keys[q]));
      kmax = max(kmax, keys[q]);
    }
  } else {
#pragma unroll
    for (int q = 0; q < EPT; ++q) kmax = max(kmax, keys[q]);
  }
  uint32_t lb = J == 1 ? kmax : (J == 2 ? k2 : 0u);
  const bool need_min = !dense || J > 2 || n - (kRowW - 1) * 64 * EPT < 64 * J;  // uniform
  uint32_t kmin1 = 0xFFFFFFFFu;  // smallest valid key - 1 (a zero key wraps to the top)
  if (need_min) {
#pragma unroll
    for (int q = 0; q < EPT; ++q) kmin1 = min(kmin1, keys[q] - 1u);
  }
  int nv = 0;  // valid keys of the wave (uniform)
  if constexpr (dense) {
    nv = wn;
  } else {
#pragma unroll
    for (int q = 0; q < EPT; ++q) nv += (int)__popcll(__ballot(keys[q] != 0u));
  }
  if (need_min) kmin1 = ~wave_max_u32(~kmin1);
  kmax = wave_max_u32(kmax);
  lb = ~wave_max_u32(~lb);
  if (lane == 0) {
    sh.wi[wave][1] = nv;
    sh.wu[wave][0] = kmin1;
    sh.wu[wave][1] = kmax;
    sh.wscan[wave] = (int)lb;
  }
  __syncthreads();
  // lane w < 16 reads wave w's values; one DPP row combines them
  const bool wl = lane < kRowW;
  int n_valid = n;
  if constexpr (!dense) {
    n_valid = __builtin_amdgcn_readlane(row16_incl_scan(wl ? sh.wi[lane][1] : 0), kRowW - 1);
  }
  kmax = row16_max_u32(wl ? sh.wu[lane][1] : 0u);
  lb = row16_min_u32(wl ? (uint32_t)sh.wscan[lane] : 0xFFFFFFFFu);
  const uint32_t kmin = need_min ? row16_min_u32(wl ? sh.wu[lane][0] : 0xFFFFFFFFu) + 1u : lb;
  const int take = min(kk, n_valid);
  const int mode = take == 0 ? 0 : (take == n_valid ? 1 : 2);

  // theta: narrow [lo, hi] (keys in it rank need-th from its top) to one key;
  // e_cnt = keys equal to theta, when the narrowing step yields it
  uint32_t theta = 0u;
  int t_eq = 0, e_cnt = -1;
  if (mode == 2) {
    uint32_t lo = max(kmin, lb), hi = kmax;  // theta is in [lo, hi], rank take from the top
    int need = take;
    // 4096-fold narrowing: 32-bit keys need at most three passes (the cap
    // only bounds the loop).  Once the range holds at most kRowFew keys,
    // they are ranked directly: wave w compares members 4w .. 4w+3 with
    // every member, and the counts meet in LDS.
    int m = n_valid;
    for (int pass = 0; pass < 4 && lo != hi; ++pass) {
      const uint32_t span = hi - lo;
      if (m <= kRowFew) {
#pragma unroll
        for (int q = 0; q < EPT; ++q) {
          const uint32_t k = keys[q];
          if (k - lo <= span) sh.mkeys[atomicAdd(&sh.mcount, 1u)] = k;
        }
        __syncthreads();
        const int mc = __builtin_amdgcn_readfirstlane((int)sh.mcount);
        const uint32_t mine = sh.mkeys[lane];  // meaningful for lane < mc
        const u32x4 k4 = *reinterpret_cast<const u32x4*>(&sh.mkeys[4 * wave]);
        int gt = 0, ge = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bool in = 4 * wave + c < mc;
          gt += in && k4[c] > mine;
          ge += in && k4[c] >= mine;
        }
        if (lane < mc && ge > 0) {
          if (gt > 0) atomicAdd(&sh.rk[lane][0], gt);
          atomicAdd(&sh.rk[lane][1], ge);
        }
        __syncthreads();
        if (wave == 0 && lane < mc) {
          const int g_ = sh.rk[lane][0], e_ = sh.rk[lane][1];
          if (g_ < need && need <= e_) {  // every such lane holds the same key
            sh.u[0] = mine;
            sh.u[1] = (uint32_t)(need - g_);
            sh.u[2] = (uint32_t)(e_ - g_);
          }
        }
        __syncthreads();
        lo = hi = __builtin_amdgcn_readfirstlane(sh.u[0]);
        need = __builtin_amdgcn_readfirstlane((int)sh.u[1]);
        e_cnt = __builtin_amdgcn_readfirstlane((int)sh.u[2]);
        break;
      }
      const int sft = max(0, 20 - (int)__builtin_clz(span | 1u));  // span >> sft < kRowBins
#pragma unroll
      for (int q = 0; q < EPT; ++q) {
        const uint32_t d = keys[q] - lo;
        if (d <= span) atomicAdd(&sh.h[d >> sft], 1u);
      }
      __syncthreads();
      uint32_t b;
      int ab;
      row_locate(sh, need, b, ab, m);
      lo += b << sft;
      const uint32_t wbin = (1u << sft) - 1u;
      hi = hi - lo > wbin ? lo + wbin : hi;
      need -= ab;
      if (lo == hi) e_cnt = m;  // the bin holds a single key value
    }
    theta = lo;
    t_eq = need;  // theta-ties to keep, in index order
  }

  // kept: key > theta (mode 1: every valid key), or one of the first t_eq
  // theta-ties in index order.  Per-wave counts from ballots.
  const bool all_ties = mode == 1 || (mode == 2 && e_cnt == t_eq);
  const uint32_t kmin_kept = mode == 1 ? 1u : theta;  // when every tie is kept
  int c_gt = 0, c_eq = 0;  // uniform
  if (all_ties) {
#pragma unroll
    for (int q = 0; q < EPT; ++q) c_gt += (int)__popcll(__ballot(keys[q] >= kmin_kept));
  } else if (mode == 2) {
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      c_gt += (int)__popcll(__ballot(keys[q] > theta));
      c_eq += (int)__popcll(__ballot(keys[q] == theta));
    }
  }
  if (lane == 0) {
    sh.wc[wave][0] = c_gt;
    sh.wc[wave][1] = c_eq;
  }
  __syncthreads();
  // lane w < 16 takes wave w: kept ties of wave w are the first of the
  // t_eq - (ties in earlier waves) still to keep; offsets are the exclusive
  // prefix of the kept counts
  int o = 0, eseen = 0, e_total = 0;
  if (all_ties) {
    const int incl = row16_incl_scan(lane < kRowW ? sh.wc[lane][0] : 0);
    o = wave ? __builtin_amdgcn_readlane(incl, wave - 1) : 0;
  } else {
    const int cg = lane < kRowW ? sh.wc[lane][0] : 0, ce = lane < kRowW ? sh.wc[lane][1] : 0;
    const int e_incl = row16_incl_scan(ce);
    const int kept = cg + max(0, min(ce, t_eq - (e_incl - ce)));
    const int k_incl = row16_incl_scan(kept);
    o = wave ? __builtin_amdgcn_readlane(k_incl, wave - 1) : 0;
    eseen = wave ? __builtin_amdgcn_readlane(e_incl, wave - 1) : 0;
    e_total = __builtin_amdgcn_readlane(e_incl, kRowW - 1);
  }
  const bool simple = all_ties || e_total <= t_eq;  // every kept key is >= kmin_kept

  // padding and count (only the last block can be partial)
  const int bs = a.block;
  int32_t* out = pool_mode ? a.pool + (int64_t)r * a.pool_stride : a.idx + (int64_t)r * a.idx_stride;
  if constexpr (pool_mode) {
    bool last_kept = false;
    if (mode != 0) {
      const uint32_t kl = s.key(n - 1);  // the highest-index block: a tie is kept iff all are
      last_kept = mode == 1 ? kl != 0u : (kl > theta || (kl == theta && simple));
    }
    const int pool_n = take * bs - (last_kept ? n * bs - ri.win_lo : 0);
    for (int i = pool_n + tid; i < a.max_blocks * bs; i += kRowT) out[i] = -1;
    if (tid == 0) a.pool_count[r] = pool_n;
  } else {
    for (int i = take + tid; i < a.k; i += kRowT) out[i] = -1;
    if (tid == 0) a.count[r] = take;
  }
  if (mode == 0) return;

  // pool rows of whole 8-entry blocks go out as two 16-byte stores
  const bool vec8 = pool_mode && bs == 8 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  auto put = [&](int j, int rank) {
    if constexpr (pool_mode) {
      const int lo = j * bs, mm = min(bs, ri.win_lo - lo);
      if (vec8 && mm == 8) {
        int32_t* o8 = out + rank * 8;
        reinterpret_cast<i32x4*>(o8)[0] = i32x4{lo, lo + 1, lo + 2, lo + 3};
        reinterpret_cast<i32x4*>(o8)[1] = i32x4{lo + 4, lo + 5, lo + 6, lo + 7};
      } else {
        for (int u = 0; u < mm; ++u) out[rank * bs + u] = lo + u;
      }
    } else {
      out[rank] = s.position(j);
    }
  };
  if (simple) {
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const bool keep = keys[q] >= kmin_kept;
      const uint64_t mk = __ballot(keep);
      if (keep) put(jw + 64 * q, o + (int)__popcll(mk & below));
      o += (int)__popcll(mk);
    }
    return;
  }
  // only some theta-ties are kept: they also need their rank among the ties
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    const uint32_t k = keys[q];
    const bool eq = k == theta;
    const uint64_t me = __ballot(eq);
    const bool keep = k > theta || (eq && eseen + (int)__popcll(me & below) < t_eq);
    const uint64_t mk = __ballot(keep);
    if (keep) put(jw + 64 * q, o + (int)__popcll(mk & below));
    o += (int)__popcll(mk);
    eseen += (int)__popcll(me);
  }
}

// Chunks of 2048 elements; when rows x chunks already gives many workgroups
// (prefill row blocks), chunks of 8192, so the per-chunk fixed work (row
// histogram, member list) is spread over 4x more elements.
template <int KIND, int CHUNK>
void run_select_chunk(const SelectArgs& a, const Ws& ws, int64_t max_n, int kk, int pool_mode,
                      hipStream_t st) {
  const int R = a.rows.n_rows;
  int64_t nchunks = (max_n + CHUNK - 1) / CHUNK;
  dim3 gc((unsigned)(nchunks > 0 ? nchunks : 1), R);
  static_assert(kHistStride % 4 == 0, "whole 16-byte vectors per row histogram");
  const int64_t n_vec = (int64_t)R * kHistStride / 4;
  hipLaunchKernelGGL(zero_hist_kernel, dim3((unsigned)((n_vec + 255) / 256)), dim3(256), 0, st, ws,
                     n_vec);
  hipLaunchKernelGGL((hist_kernel<KIND, CHUNK>), gc, dim3(kChunkT), 0, st, a, ws);
  hipLaunchKernelGGL((scan_kernel<KIND, CHUNK>), gc, dim3(kChunkT), 0, st, a, ws, kk);
  hipLaunchKernelGGL((emit_kernel<KIND, CHUNK>), gc, dim3(kChunkT), 0, st, a, ws, pool_mode);
}

template <int KIND>
void run_select(const SelectArgs& a, const Ws& ws, int64_t max_n, int kk, int pool_mode,
                hipStream_t st) {
  const int R = a.rows.n_rows;
  if (max_n <= 16 * kRowT) {
    hipLaunchKernelGGL((row_select_kernel<KIND, 16>), dim3(R), dim3(kRowT), 0, st, a, ws, kk);
    return;
  }
  if (max_n <= 32 * kRowT) {
    hipLaunchKernelGGL((row_select_kernel<KIND, 32>), dim3(R), dim3(kRowT), 0, st, a, ws, kk);
    return;
  }
  if (max_n <= 64 * kRowT) {
    hipLaunchKernelGGL((row_select_kernel<KIND, 64>), dim3(R), dim3(kRowT), 0, st, a, ws, kk);
    return;
  }
  const int64_t wgs = (int64_t)R * ((max_n + kChunk - 1) / kChunk);
  if (wgs >= 16384)
    run_select_chunk<KIND, 4 * kChunk>(a, ws, max_n, kk, pool_mode, st);
  else
    run_select_chunk<KIND, kChunk>(a, ws, max_n, kk, pool_mode, st);
}

int64_t chunk_stride(const SelectArgs& a) {
  int64_t n = a.max_elems;
  if (a.pool) n = max(n, a.beta_stride);
  return ((n + kChunk - 1) / kChunk + 15) / 16 * 16;
}

}  // namespace

size_t topk_workspace_bytes(const SelectArgs& a) {
  const int64_t R = a.rows.n_rows;
  size_t b = (size_t)R * (kHistStride + kRecWords + 2 * kCapM) * sizeof(uint32_t);
  b += (size_t)R * 2 * chunk_stride(a) * sizeof(int32_t);
  if (a.pool) b += (size_t)R * a.beta_stride * sizeof(float);
  return b;
}

// Workspace: level-1 histograms [R][kHistStride] (cleared by the call),
// per-row records, member lists, per-chunk counts, then (pool mode) block
// maxima.
hipError_t launch_topk_select(const SelectArgs& a, hipStream_t st) {
  if (a.rows.n_rows == 0) return hipSuccess;
  const int64_t R = a.rows.n_rows;
  Ws ws;
  ws.hist = reinterpret_cast<uint32_t*>(a.beta);
  ws.rec = ws.hist + R * kHistStride;
  ws.mkey = ws.rec + R * kRecWords;
  ws.midx = reinterpret_cast<int32_t*>(ws.mkey + R * kCapM);
  ws.chunk_stride = chunk_stride(a);
  ws.cgt = ws.midx + R * kCapM;
  ws.cm = ws.cgt + R * ws.chunk_stride;
  ws.beta = reinterpret_cast<float*>(ws.cm + R * ws.chunk_stride);
  if ((a.pool ? max((int64_t)a.max_elems, a.beta_stride) : a.max_elems) >
      (int64_t)kChunk * kMaxChunks)
    return hipErrorInvalidValue;
  if (a.pool) {
    dim3 g2((unsigned)((a.beta_stride + 255) / 256), a.rows.n_rows);
    hipLaunchKernelGGL(block_max_kernel, g2, dim3(256), 0, st, a, ws);
    run_select<SRC_BLOCK>(a, ws, a.beta_stride, a.max_blocks, 1, st);
  }
  if (a.k > 0) {
    // The pool holds the whole token top-k when at least k blocks are kept
    // (blocks and tokens both range over the candidates): a block left out
    // has max_blocks blocks before it in (max desc, block asc) order, and each
    // of their maxima ranks before every token of the left-out block.
    if (a.pool && a.max_blocks >= a.k)
      run_select<SRC_POOL>(a, ws, (int64_t)a.max_blocks * a.block, a.k, 0, st);
    else if (a.cand)
      run_select<SRC_TOKEN_CAND>(a, ws, a.cand_stride, a.k, 0, st);
    else
      run_select<SRC_TOKEN_FULL>(a, ws, a.max_elems, a.k, 0, st);
  }
  return hipGetLastError();
}

}  // namespace sa
