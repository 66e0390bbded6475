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
// holds channels [g*dim/4, (g+1)*dim/4); k-step ks uses its ks-th group of 8.
template <int DIM, bool FP8>
struct LaneSlice {
  static constexpr int KS = DIM / 32;
  static constexpr int BYTES = DIM / 4 * ElemTraits<FP8>::bytes;
  static constexpr int VEC = BYTES / 16;  // 16-byte vectors per lane
  u32x4 v[VEC];

  __device__ __forceinline__ void load(const char* row, int g) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row + g * BYTES);
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = __builtin_nontemporal_load(p + i);
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

// grid = (ceil(n_slots / (64*kWaves*GPW)), R); wave w scores GPW groups of 64
// consecutive slots of row blockIdx.y, 16 entries per MFMA tile.  All of a
// wave's key rows are loaded before the first MFMA: slot -> entry -> cache
// row addresses first, then every row load (unconditional, with the entry
// clamped to a visible one), so a wave keeps 4*GPW tiles of loads in flight.
template <int NMT, int DIM, bool FP8, int GPW>
__global__ __launch_bounds__(64 * kWaves) void index_score_mfma(IndexArgs a) {
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const RowInfo ri = row_info(a.rows, r);
  const bool cand_mode = a.cand != nullptr;
  const int n_slots = cand_mode ? a.cand_count[r] : ri.n_avail;
  const int wg_base = blockIdx.x * (64 * kWaves * GPW);
  if (wg_base >= n_slots) return;
  float* out = a.scores + (int64_t)r * a.score_stride;
  if (ri.n_avail == 0) {  // nothing visible: every listed candidate scores -inf
    for (int i = threadIdx.x; i < 64 * kWaves * GPW && wg_base + i < n_slots; i += 64 * kWaves)
      out[wg_base + i] = -__builtin_huge_valf();
    return;
  }
  const int32_t* cand = cand_mode ? a.cand + (int64_t)r * a.cand_stride : nullptr;
  const int wbase = wg_base + wave * 64 * GPW;

  // entries of this lane's rows (tile t of group gi: slot wbase + 64 gi + 16 t + col)
  int pos[GPW][4];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int slot = wbase + 64 * gi + 16 * t + col;
      pos[gi][t] = cand_mode ? cand[min(slot, n_slots - 1)] : slot;
    }
  constexpr int EB = ElemTraits<FP8>::bytes;
  LaneSlice<DIM, FP8> ks[GPW][4];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int pc = min(max(pos[gi][t], 0), ri.n_avail - 1);
      ks[gi][t].load(cache_row(a.k, ri.b, pc), g);
    }

  // Query slices (A operand: head = mt*16 + col) and head weights in the
  // accumulator layout (head = mt*16 + 4*g + i).
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

#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int base = wbase + 64 * gi;
    float res[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int slot = base + 16 * t + col;
      const int p = pos[gi][t];
      const bool valid = slot < n_slots && p >= 0 && p < ri.n_avail;
      float part = 0.0f;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma_slice<DIM>(qs[mt], ks[gi][t], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) part = fmaf(wv[mt][i], fmaxf(acc[i], 0.0f), part);
      }
      part = xor16_32_sum(part);
      res[t] = valid ? part : -__builtin_huge_valf();
    }
    // lane l stores the result of slot base + l (tile l/16, column l%16)
    const float mine = g == 0 ? res[0] : g == 1 ? res[1] : g == 2 ? res[2] : res[3];
    if (base + lane < n_slots) out[base + lane] = mine;
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
  if (pos >= 0 && pos < ri.n_avail) {
    const float* kr = reinterpret_cast<const float*>(cache_row(a.k, ri.b, pos));
    s = 0.0f;
    for (int h = 0; h < a.n_heads; ++h) {
      float d = 0.0f;
      for (int c = 0; c < a.dim; ++c) d = fmaf(smem[h * a.dim + c], kr[c], d);
      s = fmaf(smem[HD + h], fmaxf(d, 0.0f), s);
    }
  }
  a.scores[(int64_t)r * a.score_stride + slot] = s;
}

template <int NMT, int DIM, bool FP8>
hipError_t launch_mfma(const IndexArgs& a, hipStream_t s) {
  // Rows of keys per lane held at once: 4 tiles x GPW groups; wide keys
  // (dim 128) keep one group per wave so the loads fit the register file.
  constexpr int GPW = DIM == 64 ? 2 : 1;
  const int per_wg = 64 * kWaves * GPW;
  dim3 grid((a.n_slots + per_wg - 1) / per_wg, a.rows.n_rows);
  hipLaunchKernelGGL((index_score_mfma<NMT, DIM, FP8, GPW>), grid, dim3(64 * kWaves), 0, s, a);
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
  if (a.dim == 64) return fp8 ? dispatch_heads<64, true>(a, s) : dispatch_heads<64, false>(a, s);
  return fp8 ? dispatch_heads<128, true>(a, s) : dispatch_heads<128, false>(a, s);
}

}  // namespace sa
