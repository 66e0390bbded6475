// Window + top-k selection and the block-max candidate pool on gfx950.
//
// Token mode ("HySparse2", section 7.2): the candidates of a row are the
// visible entries outside the forced window; keep the first min(k, n) in the
// order (score desc, index asc).  Pool mode ("CSA, HCA and CSA2", section
// 3.2, Hierarchical Sparse Indexer): every aligned block of `block` entries is
// scored by its maximum over visible members, the first max_blocks blocks in
// (max desc, block asc) order are kept and their members form the pool.
//
// One workgroup per row.  Scores become order-preserving uint32 keys (-0
// folded onto +0).  The kept set is {key > theta} plus the elements with
// key == theta up to index jstar, where (theta, jstar) is the take-th element
// of the total order.  It is found without sorting:
//   1. each thread holds the keys of a contiguous index range in registers;
//   2. a 2048-bin histogram linear in score over the row's [min, max] (a
//      monotone map that spreads real score distributions over many bins and
//      keeps LDS atomic contention low) locates the bin of the take-th key;
//   3. the few elements of that bin are gathered into LDS and ranked exactly
//      by (key desc, index asc); a crowded bin (heavy ties) falls back to an
//      exact 8-bit radix refinement restricted to that bin;
//   4. an ordered compaction (block prefix sums over the contiguous ranges)
//      writes the kept indices ascending.
// The output depends only on the total order, never on thread timing.
#include "kernels.hpp"

namespace sa {

namespace {

constexpr int kBins = 2048;
constexpr int kCap = 2048;      // LDS slots (threshold-bin elements, kept blocks)
constexpr int kRankMax = 512;   // largest threshold bin ranked by direct comparison

// Float value of an order-preserving key (inverse of order_key).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

enum { SRC_TOKEN_FULL = 0, SRC_TOKEN_CAND = 1, SRC_BLOCK = 2, SRC_POOL = 3 };

// The elements being ranked (KIND fixes how an element's key is formed).
// key() == 0 marks an element that can never be kept: every real score maps
// to a key >= order_key(-inf) > 0.
template <int KIND>
struct Src {
  const float* sc;      // this row's scores
  const int32_t* list;  // candidate list (SRC_TOKEN_CAND) or pool (SRC_POOL)
  int n;                // elements
  int win_lo;           // kept tokens must lie below this entry
  int n_avail;
  int block;

  __device__ __forceinline__ uint32_t key(int j) const {
    if constexpr (KIND == SRC_TOKEN_FULL) {
      return order_key(sc[j]);
    } else if constexpr (KIND == SRC_TOKEN_CAND) {
      const int p = list[j];
      return (p >= 0 && p < win_lo) ? order_key(sc[j]) : 0u;
    } else if constexpr (KIND == SRC_POOL) {
      const int p = list[j];
      return (p >= 0 && p < win_lo) ? order_key(sc[p]) : 0u;
    } else {  // SRC_BLOCK: sc holds the row's block maxima
      return order_key(sc[j]);
    }
  }
  static constexpr bool may_be_invalid() {
    return KIND == SRC_TOKEN_CAND || KIND == SRC_POOL;
  }
  // value written for a kept token element
  __device__ __forceinline__ int position(int j) const {
    if constexpr (KIND == SRC_TOKEN_FULL) return j;
    else return list[j];
  }
};

template <int NT>
struct Shared {
  uint32_t hist[kBins];
  uint32_t ckey[kCap];
  int32_t cidx[kCap];
  int cnt[NT];  // per (slot, wave) counts of an ordered pass (KPT * NT/64 <= NT)
  int scan[NT / 64];
  uint32_t u[8];
};

// Exclusive prefix sum over the workgroup; *total receives the sum.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* total, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int wv = lane < NT / 64 ? sh[lane] : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(wv, o, 64);
      if (lane >= o) wv += y;
    }
    if (lane < NT / 64) sh[lane] = wv;
  }
  __syncthreads();
  const int base = wave ? sh[wave - 1] : 0;
  *total = sh[NT / 64 - 1];
  __syncthreads();
  return base + x - v;
}

template <int NT>
__device__ __forceinline__ uint32_t block_reduce_max(uint32_t v, int* sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sh[wave] = (int)v;
  __syncthreads();
  uint32_t r = 0;
  for (int i = 0; i < NT / 64; ++i) r = max(r, (uint32_t)sh[i]);
  __syncthreads();
  return r;
}

// One histogram increment per element, with a single atomic when the whole
// wave hits one bin (massive ties).
__device__ __forceinline__ void hist_add(uint32_t* hist, bool v, int bin) {
  const uint64_t vm = __ballot(v);
  if (vm == 0) return;
  const int lead = __ffsll((unsigned long long)vm) - 1;
  const int bl = __shfl(bin, lead, 64);
  const uint64_t sm = __ballot(v && bin == bl);
  if (sm == vm) {
    if ((int)(threadIdx.x & 63) == lead) atomicAdd(&hist[bl], (uint32_t)__popcll(sm));
  } else if (v) {
    atomicAdd(&hist[bin], 1u);
  }
}

struct Pick {
  uint32_t theta;  // keep key > theta ...
  int jstar;       // ... and key == theta with index <= jstar
  int take;        // number kept
};

// Elements are striped over the workgroup: chunk c holds NT*KPT consecutive
// elements and thread t owns elements c*NT*KPT + i*NT + t (i < KPT), so every
// load instruction of a wave reads 64 consecutive scores.  When the row fits
// in one chunk the keys stay in registers (kc[]); otherwise they are
// recomputed from memory in every pass.
template <int NT, int KPT, class S>
struct Range {
  int n, nchunks;
  bool cached;
  uint32_t kc[KPT];

  __device__ __forceinline__ void init(const S& s) {
    n = s.n;
    nchunks = (n + NT * KPT - 1) / (NT * KPT);
    cached = nchunks <= 1;
    if (cached) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int j = i * NT + (int)threadIdx.x;
        kc[i] = j < n ? s.key(j) : 0u;
        // bound the loads in flight (a block key reads `block` scores)
        if ((i & 7) == 7) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // f(index, key, in_range) for every owned slot, in increasing index order
  // per thread; the trip count is wave-uniform, so f may use wave collectives.
  template <class F>
  __device__ __forceinline__ void visit(const S& s, F f) const {
    if (cached) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int j = i * NT + (int)threadIdx.x;
        f(j, kc[i], j < n);
      }
    } else {
      for (int c = 0; c < nchunks; ++c) {
#pragma unroll 4
        for (int i = 0; i < KPT; ++i) {
          const int j = c * NT * KPT + i * NT + (int)threadIdx.x;
          const bool in = j < n;
          f(j, in ? s.key(j) : 0u, in);
        }
      }
    }
  }
  // Calls emit(index, rank) for every owned element with sel(index, key)
  // true, where rank is its position among all selected elements in
  // increasing index order.  Returns the number selected.
  template <class Sel, class Emit>
  __device__ __forceinline__ int ordered(const S& s, Sel sel, Emit emit, int* cnt_lds,
                                         int* scan_sh) const {
    if (cached) return ordered_chunk<true>(s, 0, 0, sel, emit, cnt_lds, scan_sh);
    int running = 0;
    for (int c = 0; c < nchunks; ++c)
      running = ordered_chunk<false>(s, c, running, sel, emit, cnt_lds, scan_sh);
    return running;
  }

  template <bool CACHED, class Sel, class Emit>
  __device__ __forceinline__ int ordered_chunk(const S& s, int c, int running, Sel sel,
                                               Emit emit, int* cnt_lds, int* scan_sh) const {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    uint32_t flags = 0u;  // selection bits of slots 0..31 (recomputed past 32)
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int j = c * NT * KPT + i * NT + (int)threadIdx.x;
      const bool in = j < n;
      uint32_t key;
      if (CACHED)
        key = kc[i];
      else
        key = in ? s.key(j) : 0u;
      const bool me = in && sel(j, key);
      if (i < 32 && me) flags |= 1u << i;
      const uint64_t m = __ballot(me);
      if (lane == 0) cnt_lds[i * NW + wave] = __popcll(m);
    }
    __syncthreads();
    int total;
    const int v = (int)threadIdx.x < KPT * NW ? cnt_lds[threadIdx.x] : 0;
    const int ex = block_excl_scan<NT>(v, &total, scan_sh);
    if ((int)threadIdx.x < KPT * NW) cnt_lds[threadIdx.x] = ex;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int j = c * NT * KPT + i * NT + (int)threadIdx.x;
      bool me;
      if (i < 32) {
        me = (flags >> i) & 1u;
      } else {
        const bool in = j < n;
        uint32_t key;
        if (CACHED)
          key = kc[i];
        else
          key = in ? s.key(j) : 0u;
        me = in && sel(j, key);
      }
      const uint64_t m = __ballot(me);
      if (me) emit(j, running + cnt_lds[i * NW + wave] + __popcll(m & below));
    }
    __syncthreads();
    return running + total;
  }
};

template <int NT, int KPT, class S>
__device__ __forceinline__ Pick select_top(const S& s, const Range<NT, KPT, S>& rg, int k,
                                          Shared<NT>& sh) {
  Pick pk;
  pk.theta = 0u;
  pk.jstar = -1;
  int n_valid = s.n;
  if constexpr (S::may_be_invalid()) {
    int c = 0;
    rg.visit(s, [&](int, uint32_t key, bool in) { c += in && key != 0u; });
    block_excl_scan<NT>(c, &n_valid, sh.scan);
  }
  pk.take = min(k, n_valid);
  if (pk.take == 0 || pk.take == n_valid) return pk;  // none, or every valid element

  // key range of the valid elements
  uint32_t kmax = 0u, kmin_inv = 0u;  // max of key and of ~key over valid keys
  rg.visit(s, [&](int, uint32_t key, bool in) {
    if (in && key != 0u) {
      kmax = max(kmax, key);
      kmin_inv = max(kmin_inv, ~key);
    }
  });
  kmax = block_reduce_max<NT>(kmax, sh.scan);
  const uint32_t kmin = ~block_reduce_max<NT>(kmin_inv, sh.scan);
  // Linear bins in score VALUE over [min, max]: x -> (x - min) * scale is
  // monotone non-decreasing in floating point, so bins respect the order and
  // equal scores share a bin.  (Bins linear in key space would put a range
  // starting at 0 into a handful of bins.)  A non-finite span maps every
  // element to bin 0 and the exact refinement below takes over.
  const float xmin = key_value(kmin), xmax = key_value(kmax);
  float span = xmax - xmin;
  const float scale = (span > 0.0f && span < 3.0e38f) ? (float)kBins / span : 0.0f;
  auto bin_of = [&](uint32_t key) {
    const float t = (key_value(key) - xmin) * scale;
    return min(kBins - 1, (int)t);
  };

  for (int i = threadIdx.x; i < kBins; i += NT) sh.hist[i] = 0u;
  __syncthreads();
  rg.visit(s, [&](int, uint32_t key, bool in) {
    const bool v = in && key != 0u;
    hist_add(sh.hist, v, v ? bin_of(key) : 0);
  });
  __syncthreads();

  // Locate the bin holding the take-th key, scanning bins from the top.
  constexpr int BPT = kBins / NT;
  {
    const int hi = kBins - (int)threadIdx.x * BPT;  // bins [hi - BPT, hi)
    int mine = 0;
#pragma unroll
    for (int b = 0; b < BPT; ++b) mine += (int)sh.hist[hi - 1 - b];
    int tot;
    const int above = block_excl_scan<NT>(mine, &tot, sh.scan);
    if (above < pk.take && pk.take <= above + mine) {
      int acc = above;
      for (int b = 0; b < BPT; ++b) {
        const int c = (int)sh.hist[hi - 1 - b];
        if (acc + c >= pk.take) {
          sh.u[0] = (uint32_t)(hi - 1 - b);
          sh.u[1] = (uint32_t)acc;
          break;
        }
        acc += c;
      }
    }
    __syncthreads();
  }
  const int bstar = (int)sh.u[0];
  const int need = pk.take - (int)sh.u[1];  // rank (1-based) inside bin bstar
  const int m = (int)sh.hist[bstar];

  // Recompute bins from laundered copies of the map below, so the compiler
  // does not keep every element's bin live across passes.
  float scale_b = scale, xmin_b = xmin;
  asm volatile("" : "+v"(scale_b), "+v"(xmin_b));
  auto bin_again = [&](uint32_t key) {
    const float t = (key_value(key) - xmin_b) * scale_b;
    return min(kBins - 1, (int)t);
  };
  if (m <= kRankMax) {
    // gather the bin's elements into LDS and rank them exactly
    if (threadIdx.x == 0) sh.u[2] = 0u;
    __syncthreads();
    rg.visit(s, [&](int j, uint32_t key, bool in) {
      if (in && key != 0u && bin_again(key) == bstar) {
        const uint32_t slot = atomicAdd(&sh.u[2], 1u);
        sh.ckey[slot] = key;
        sh.cidx[slot] = j;
      }
    });
    __syncthreads();
    for (int i = threadIdx.x; i < m; i += NT) {
      const uint32_t ki = sh.ckey[i];
      const int ji = sh.cidx[i];
      int rank = 0;
      for (int l = 0; l < m; ++l) {
        const uint32_t kl = sh.ckey[l];
        rank += kl > ki || (kl == ki && sh.cidx[l] < ji);
      }
      if (rank == need - 1) {
        sh.u[3] = ki;
        sh.u[4] = (uint32_t)ji;
      }
    }
    __syncthreads();
    pk.theta = sh.u[3];
    pk.jstar = (int)sh.u[4];
    __syncthreads();
    return pk;
  }

  // Crowded bin: exact 8-bit radix refinement restricted to it.
  uint32_t prefix = 0u, pmask = 0u;
  int remaining = need;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += NT) sh.hist[i] = 0u;
    __syncthreads();
    rg.visit(s, [&](int, uint32_t key, bool in) {
      const bool v = in && key != 0u && bin_again(key) == bstar && (key & pmask) == prefix;
      hist_add(sh.hist, v, v ? (int)((key >> shift) & 255u) : 0);
    });
    __syncthreads();
    if (threadIdx.x == 0) {
      int above = 0, d = 255;
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
    pmask |= 255u << shift;
    __syncthreads();
  }
  pk.theta = prefix;
  // the remaining-th element equal to theta, in index order
  rg.ordered(
      s, [&](int, uint32_t key) { return key == prefix; },
      [&](int j, int rank) {
        if (rank == remaining - 1) sh.u[4] = (uint32_t)j;
      },
      sh.cnt, sh.scan);
  __syncthreads();
  pk.jstar = (int)sh.u[4];
  __syncthreads();
  return pk;
}

// beta[r][j] = max of the visible scores of block j (one thread per block).
__global__ __launch_bounds__(256) void block_max_kernel(SelectArgs a) {
  const int r = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  const RowInfo ri = row_info(a.rows, r);
  const int nb = (ri.n_avail + a.block - 1) / a.block;
  if (j >= nb) return;
  const float* sc = a.scores + (int64_t)r * a.score_stride;
  const int lo = j * a.block, hi = min(lo + a.block, ri.n_avail);
  float m = sc[lo];
  for (int s = lo + 1; s < hi; ++s) m = fmaxf(m, sc[s]);
  a.beta[(int64_t)r * a.beta_stride + j] = m;
}

// Block-max pool of one row per workgroup, ranking the block maxima.
template <int NT, int KPT>
__global__ __launch_bounds__(NT) void pool_select_kernel(SelectArgs a) {
  __shared__ Shared<NT> sh;
  using S = Src<SRC_BLOCK>;
  const int r = blockIdx.x;
  const RowInfo ri = row_info(a.rows, r);
  S s;
  s.sc = a.beta + (int64_t)r * a.beta_stride;
  s.list = nullptr;
  s.n = (ri.n_avail + a.block - 1) / a.block;
  s.win_lo = ri.win_lo;
  s.n_avail = ri.n_avail;
  s.block = a.block;
  Range<NT, KPT, S> rg;
  rg.init(s);
  const Pick pk = select_top<NT, KPT>(s, rg, a.max_blocks, sh);
  // kept blocks, ascending, into LDS (max_blocks <= kCap), then expanded
  const int nsel = rg.ordered(
      s,
      [&](int j, uint32_t key) {
        return pk.take > 0 && (key > pk.theta || (key == pk.theta && j <= pk.jstar));
      },
      [&](int j, int rank) { sh.cidx[rank] = j; }, sh.cnt, sh.scan);
  __syncthreads();
  int32_t* out = a.pool + (int64_t)r * a.pool_stride;
  const int bs = a.block;
  // only the last block of the domain can be partial, and it is kept last
  const int last_blk = s.n - 1;
  const int deficit =
      (nsel > 0 && sh.cidx[nsel - 1] == last_blk) ? (last_blk + 1) * bs - ri.n_avail : 0;
  const int pool_n = nsel * bs - deficit;
  for (int i = threadIdx.x; i < a.max_blocks * bs; i += NT)
    out[i] = i < pool_n ? sh.cidx[i / bs] * bs + i % bs : -1;
  if (threadIdx.x == 0) a.pool_count[r] = pool_n;
}

// Token top-k of one row per workgroup.  KIND = SRC_TOKEN_FULL (visible
// entries outside the window), SRC_TOKEN_CAND (a candidate list) or SRC_POOL
// (the block-max pool of the same scores: with no window and a pool of at
// least k blocks the token top-k lies inside the pool -- a block ranked above
// the block of a kept token has a maximum that itself ranks above that token,
// so at most k-1 blocks rank above it -- and ranking only the pool gives the
// same set).
template <int KIND, int NT, int KPT>
__global__ __launch_bounds__(NT) void token_select_kernel(SelectArgs a) {
  __shared__ Shared<NT> sh;
  using S = Src<KIND>;
  const int r = blockIdx.x;
  const RowInfo ri = row_info(a.rows, r);
  S s;
  s.sc = a.scores + (int64_t)r * a.score_stride;
  s.win_lo = ri.win_lo;
  s.n_avail = ri.n_avail;
  s.block = 0;
  if constexpr (KIND == SRC_POOL) {
    s.list = a.pool + (int64_t)r * a.pool_stride;
    s.n = a.pool_count[r];
  } else if constexpr (KIND == SRC_TOKEN_CAND) {
    s.list = a.cand + (int64_t)r * a.cand_stride;
    s.n = a.cand_count[r];
  } else {
    s.list = nullptr;
    s.n = ri.win_lo;
  }
  Range<NT, KPT, S> rg;
  rg.init(s);
  const Pick pk = select_top<NT, KPT>(s, rg, a.k, sh);
  int32_t* out = a.idx + (int64_t)r * a.idx_stride;
  rg.ordered(
      s,
      [&](int j, uint32_t key) {
        return pk.take > 0 && key != 0u && (key > pk.theta || (key == pk.theta && j <= pk.jstar));
      },
      [&](int j, int rank) { out[rank] = s.position(j); }, sh.cnt, sh.scan);
  for (int i = pk.take + threadIdx.x; i < a.k; i += NT) out[i] = -1;
  if (threadIdx.x == 0) a.count[r] = pk.take;
}

template <int NT, int KPT>
void launch_all(const SelectArgs& a, hipStream_t s) {
  dim3 grid(a.rows.n_rows);
  if (a.pool) {
    dim3 g2((unsigned)((a.beta_stride + 255) / 256), a.rows.n_rows);
    hipLaunchKernelGGL(block_max_kernel, g2, dim3(256), 0, s, a);
    hipLaunchKernelGGL((pool_select_kernel<NT, KPT>), grid, dim3(NT), 0, s, a);
  }
  if (a.k <= 0) return;
  if (a.pool && a.rows.window == 0 && a.max_blocks >= a.k)
    hipLaunchKernelGGL((token_select_kernel<SRC_POOL, NT, KPT>), grid, dim3(NT), 0, s, a);
  else if (a.cand)
    hipLaunchKernelGGL((token_select_kernel<SRC_TOKEN_CAND, NT, KPT>), grid, dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((token_select_kernel<SRC_TOKEN_FULL, NT, KPT>), grid, dim3(NT), 0, s, a);
}

}  // namespace

size_t topk_workspace_bytes(const SelectArgs& a) {
  if (!a.pool) return 0;
  const int64_t nb = (a.score_stride + a.block - 1) / a.block;
  const int64_t stride = (nb + 63) / 64 * 64;
  return (size_t)a.rows.n_rows * stride * sizeof(float);
}

hipError_t launch_topk_select(const SelectArgs& a, hipStream_t s) {
  if (a.rows.n_rows == 0) return hipSuccess;
  int64_t n = a.max_elems;
  if (a.pool) {
    const int64_t nb = a.beta_stride;
    const int64_t pool_tokens = (int64_t)a.max_blocks * a.block;
    n = nb;
    if (a.k > 0 && a.rows.window == 0 && a.max_blocks >= a.k) n = nb > pool_tokens ? nb : pool_tokens;
    else if (a.k > 0) n = n > a.max_elems ? n : a.max_elems;
  }
  if (n <= 256 * 16)
    launch_all<256, 16>(a, s);
  else
    launch_all<1024, 32>(a, s);
  return hipGetLastError();
}

}  // namespace sa
