// Window + top-k selection and the block-max candidate pool on gfx950.
//
// Token mode ("HySparse2", section 7.2): the candidates of a row are the
// visible entries outside the forced window; keep the first min(k, n) in the
// order (score desc, index asc).  Pool mode ("CSA, HCA and CSA2", section
// 3.2, Hierarchical Sparse Indexer): every aligned block of `block` entries is
// scored by its maximum over visible members, the first max_blocks blocks in
// (max desc, block asc) order are kept and their members form the pool.
//
// One workgroup per (row, mode).  Scores become order-preserving uint32 keys
// (-0 folded onto +0).  The kept set is {key > theta} plus the first `need`
// elements with key == theta in index order, where theta, the take-th largest
// key, comes from a 4-pass 8-bit radix select over LDS histograms.  A final
// ordered compaction (block-wide prefix sums over contiguous index ranges)
// writes the kept indices ascending, so the output is fully determined by the
// total order and needs no sort.
#include "kernels.hpp"

namespace sa {

namespace {

enum { SRC_TOKEN_FULL = 0, SRC_TOKEN_CAND = 1, SRC_BLOCK = 2 };

struct Src {
  const float* sc;       // this row's scores
  const int32_t* cand;   // this row's candidate list (candidate mode)
  int n_elem;            // elements to rank
  int win_lo;            // candidates must lie below this entry
  int n_avail;           // visible entries
  int block;             // block size (pool mode)
  int kind;

  // key 0 marks an element that can never be kept (every real score maps to a
  // key >= order_key(-inf) > 0).
  __device__ __forceinline__ uint32_t key(int j) const {
    if (kind == SRC_TOKEN_FULL) return order_key(sc[j]);
    if (kind == SRC_TOKEN_CAND) {
      int p = cand[j];
      return (p >= 0 && p < win_lo) ? order_key(sc[j]) : 0u;
    }
    int lo = j * block, hi = min(lo + block, n_avail);
    float m = sc[lo];
    for (int s = lo + 1; s < hi; ++s) m = fmaxf(m, sc[s]);
    return order_key(m);
  }
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
__global__ __launch_bounds__(NT) void topk_select_kernel(SelectArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ int scan_sh[NT / 64];
  __shared__ uint32_t sh_u[4];

  const int r = blockIdx.x;
  const bool pool_mode = blockIdx.y == 1;
  if (!pool_mode && a.k <= 0) return;
  if (pool_mode && a.pool == nullptr) return;

  const RowInfo ri = row_info(a.rows, r);
  Src src;
  src.sc = a.scores + (int64_t)r * a.score_stride;
  src.cand = a.cand ? a.cand + (int64_t)r * a.cand_stride : nullptr;
  src.win_lo = ri.win_lo;
  src.n_avail = ri.n_avail;
  src.block = a.block;
  if (pool_mode) {
    src.kind = SRC_BLOCK;
    src.n_elem = (ri.n_avail + a.block - 1) / a.block;
  } else if (a.cand) {
    src.kind = SRC_TOKEN_CAND;
    src.n_elem = a.cand_count[r];
  } else {
    src.kind = SRC_TOKEN_FULL;
    src.n_elem = ri.win_lo;
  }
  const int kk = pool_mode ? a.max_blocks : a.k;
  const int n = src.n_elem;
  const int per = (n + NT - 1) / NT;
  const int j0 = min(n, (int)threadIdx.x * per), j1 = min(n, j0 + per);

  // number of valid elements
  int n_valid = n;
  if (src.kind == SRC_TOKEN_CAND) {
    int c = 0;
    for (int j = j0; j < j1; ++j) c += src.key(j) != 0u;
    block_excl_scan<NT>(c, &n_valid, scan_sh);
  }
  const int take = min(kk, n_valid);

  uint32_t theta = 0u;  // keep key > theta, plus ties up to index jstar
  int jstar = -1;
  if (take > 0 && take < n_valid) {
    uint32_t prefix = 0u, pmask = 0u;
    int remaining = take;  // rank (1-based, from the top) still to locate
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0u;
      __syncthreads();
      for (int j = j0; j < j1; ++j) {
        uint32_t key = src.key(j);
        if (key != 0u && (key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        int above = 0, d = 255;
        for (; d > 0; --d) {
          int c = (int)hist[d];
          if (above + c >= remaining) break;
          above += c;
        }
        sh_u[0] = (uint32_t)d;
        sh_u[1] = (uint32_t)above;
      }
      __syncthreads();
      const uint32_t d = sh_u[0];
      remaining -= (int)sh_u[1];
      prefix |= d << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    theta = prefix;
    // the remaining-th element equal to theta, in index order
    int ties = 0;
    for (int j = j0; j < j1; ++j) ties += src.key(j) == theta;
    int tot;
    const int before = block_excl_scan<NT>(ties, &tot, scan_sh);
    if (before < remaining && remaining <= before + ties) {
      int c = before;
      for (int j = j0; j < j1; ++j) {
        if (src.key(j) == theta && ++c == remaining) {
          sh_u[2] = (uint32_t)j;
          break;
        }
      }
    }
    __syncthreads();
    jstar = (int)sh_u[2];
  }

  // Ordered compaction of the kept elements.
  int mine = 0;
  if (take > 0)
    for (int j = j0; j < j1; ++j) {
      uint32_t key = src.key(j);
      mine += key > theta || (key == theta && j <= jstar);
    }
  int total;
  int off = block_excl_scan<NT>(mine, &total, scan_sh);

  if (!pool_mode) {
    int32_t* out = a.idx + (int64_t)r * a.idx_stride;
    if (take > 0)
      for (int j = j0; j < j1; ++j) {
        uint32_t key = src.key(j);
        if (key > theta || (key == theta && j <= jstar))
          out[off++] = src.kind == SRC_TOKEN_CAND ? src.cand[j] : j;
      }
    for (int i = take + threadIdx.x; i < a.k; i += NT) out[i] = -1;
    if (threadIdx.x == 0) a.count[r] = take;
  } else {
    int32_t* out = a.pool + (int64_t)r * a.pool_stride;
    const int bs = a.block;
    int members = 0;
    if (take > 0)
      for (int j = j0; j < j1; ++j) {
        uint32_t key = src.key(j);
        if (key > theta || (key == theta && j <= jstar)) {
          const int lo = j * bs, m = min(bs, ri.n_avail - lo);
          for (int u = 0; u < m; ++u) out[off * bs + u] = lo + u;
          members += m;
          ++off;
        }
      }
    int pool_n;
    block_excl_scan<NT>(members, &pool_n, scan_sh);
    for (int i = pool_n + threadIdx.x; i < a.max_blocks * bs; i += NT) out[i] = -1;
    if (threadIdx.x == 0) a.pool_count[r] = pool_n;
  }
}

}  // namespace

hipError_t launch_topk_select(const SelectArgs& a, hipStream_t s) {
  if (a.rows.n_rows == 0) return hipSuccess;
  dim3 grid(a.rows.n_rows, a.pool ? 2 : 1);
  if (a.max_elems > 8192)
    hipLaunchKernelGGL(topk_select_kernel<1024>, grid, dim3(1024), 0, s, a);
  else
    hipLaunchKernelGGL(topk_select_kernel<256>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sa
