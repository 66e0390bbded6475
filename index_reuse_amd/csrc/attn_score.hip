// Selection score of a full-attention layer on gfx950.
//
// score[r][s] = sum over query sets i and query heads h of
//               exp(scale * q[i][r][h] . K[s][g(h)] - lse[i][r][h])
// for every visible entry s: the probability each head gives s in dense
// attention over the row's visible entries (lse is that attention's
// log-normaliser), summed over heads ("HySparse2", appendix A.1: the FA layer
// runs full attention and picks the important positions from its own
// attention scores; "Lecture 10", section 5.2: the per-position target is
// the main attention summed over heads).
//
// BF16 keys run on MFMA with one KV head per wave: the query rows of that
// head (every query set) sit on the M axis of v_mfma_f32_16x16x32_bf16 and 16
// entries on N, so each lane ends up with 4 heads' logits of one entry; the
// exponentials are summed in the lane, then across the four lane groups, and
// the KV heads' sums meet in LDS.  The waves of a workgroup cover the KV
// heads of the same entries, so each cache row is read from HBM once, whole.
// F32 keys use a plain loop (one thread per entry).
#include "kernels.hpp"

namespace sa {

namespace {

// One lane's slice of a row for the MFMA (lane group g holds the 16-byte
// pieces [64 i + 16 g, +16) of the row's DIM bf16 channels), as in the
// indexer: queries and keys share the mapping, so every k-step contracts
// the same channels on both operands.
template <int DIM>
struct Slice {
  static constexpr int VEC = DIM / 32;  // 16-byte vectors per lane
  u32x4 v[VEC];
  __device__ __forceinline__ void load(const char* row, int g) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row);
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = __builtin_nontemporal_load(p + 4 * i + g);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = u32x4{0u, 0u, 0u, 0u};
  }
};

constexpr int kScoreWaves = 8;  // waves per workgroup: hkv (dividing 8) x entry sub-ranges

// grid = (ceil(n_slots / (64 gpw sub)), R), sub = 8 / hkv; wave w takes KV
// head w % hkv and the w / hkv-th run of 64 gpw consecutive entries of the
// workgroup.
template <int DIM>
__global__ __launch_bounds__(64 * kScoreWaves) void attn_score_mfma(ScoreArgs a, int gpw, int sub) {
  __shared__ float red[kScoreWaves * 64];  // [wave][lane]: one 64-entry group's partial sums
  const int r = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, gq = lane >> 4;
  const int hkv = a.hkv;
  const int g = wave % hkv, sb = wave / hkv;
  const RowInfo ri = row_info(a.rows, r);
  const int n = ri.n_avail;
  const int wg_base = blockIdx.x * 64 * gpw * sub;
  if (wg_base >= n) return;  // the whole workgroup leaves together
  const int base = wg_base + sb * 64 * gpw;

  // A operand: query row m = col of this KV head (m = set * G + head in the
  // group), zero past Mq; lse of accumulator row 4 gq + i in log2 units,
  // +inf past Mq so those rows add exp2(-inf) = 0
  const int G = a.hq / hkv, Mq = a.n_qsets * G;
  Slice<DIM> qs;
  if (col < Mq) {
    const int set = col / G, h = g * G + col % G;
    qs.load(reinterpret_cast<const char*>(a.q) +
                (((int64_t)set * a.rows.n_rows + r) * a.hq + h) * DIM * 2, gq);
  } else {
    qs.zero();
  }
  float lse2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * gq + i;
    if (m < Mq) {
      const int set = m / G, h = g * G + m % G;
      lse2[i] = a.lse[((int64_t)set * a.rows.n_rows + r) * a.hq + h] * kLog2e;
    } else {
      lse2[i] = __builtin_huge_valf();
    }
  }
  const int64_t head_off = (int64_t)g * DIM * 2;
  auto load_group = [&](int gi, Slice<DIM> (&ks)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int e = min(base + 64 * gi + 16 * t + col, n - 1);  // clamped: unconditional loads
      ks[t].load(cache_row(a.k, ri.b, e) + head_off, gq);
    }
  };
  float* out = a.scores + (int64_t)r * a.score_stride;
  Slice<DIM> buf[2][4];
  load_group(0, buf[0]);
  auto score_group = [&](int gi, const Slice<DIM> (&ks)[4]) {
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks_ = 0; ks_ < Slice<DIM>::VEC; ++ks_)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qs.v[ks_]),
                                                         __builtin_bit_cast(bf16x8, ks[t].v[ks_]),
                                                         acc[t], 0, 0, 0);
    float ps[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) p += __builtin_amdgcn_exp2f(acc[t][i] * a.scale_log2 - lse2[i]);
      ps[t] = p;
    }
    // lane l: entry base + 64 gi + l, summed over this KV head's rows
    return sum4_transposed(ps[0], ps[1], ps[2], ps[3]);
  };
  // the KV heads' sums of group gi meet in LDS; wave (sb, 0) adds and stores
  auto finish = [&](int gi, float v) {
    red[wave * 64 + lane] = v;
    __syncthreads();
    if (g == 0) {
      float s = v;
      for (int gg = 1; gg < hkv; ++gg) s += red[(sb * hkv + gg) * 64 + lane];
      const int e = base + 64 * gi + lane;
      if (e < n) out[e] = s;
    }
    __syncthreads();
  };
  // Groups past the row are scored on clamped entries and never stored; the
  // loop runs gpw (even, or 1) times in every wave so the barriers match.
  // Two groups per iteration keep the register buffer index static.
  if (gpw == 1) {
    finish(0, score_group(0, buf[0]));
    return;
  }
  for (int gi = 0; gi < gpw; gi += 2) {
    load_group(gi + 1, buf[1]);
    const float v0 = score_group(gi, buf[0]);
    if (gi + 2 < gpw) load_group(gi + 2, buf[0]);
    finish(gi, v0);
    const float v1 = score_group(gi + 1, buf[1]);
    finish(gi + 1, v1);
  }
}

// F32 keys: one thread per (row, entry); query rows in LDS.
__global__ __launch_bounds__(256) void attn_score_f32(ScoreArgs a) {
  extern __shared__ float qsh[];  // [n_qsets * hq][dqk], then lse [n_qsets * hq]
  const int r = blockIdx.y;
  const RowInfo ri = row_info(a.rows, r);
  const int n = ri.n_avail;
  const int s = blockIdx.x * 256 + threadIdx.x;
  if ((int)(blockIdx.x * 256) >= n) return;
  const int nq = a.n_qsets * a.hq;
  for (int i = threadIdx.x; i < nq * a.dqk; i += 256) {
    const int qi = i / a.dqk, c = i % a.dqk;
    const int set = qi / a.hq, h = qi % a.hq;
    qsh[i] = reinterpret_cast<const float*>(a.q)[(((int64_t)set * a.rows.n_rows + r) * a.hq + h) * a.dqk + c];
  }
  for (int i = threadIdx.x; i < nq; i += 256) {
    const int set = i / a.hq, h = i % a.hq;
    qsh[nq * a.dqk + i] = a.lse[((int64_t)set * a.rows.n_rows + r) * a.hq + h] * kLog2e;
  }
  __syncthreads();
  if (s >= n) return;
  const char* row = cache_row(a.k, ri.b, s);
  const int G = a.hq / a.hkv;
  float tot = 0.f;
  for (int qi = 0; qi < nq; ++qi) {
    const int g = (qi % a.hq) / G;
    const float* kr = reinterpret_cast<const float*>(row) + g * a.dqk;
    float d = 0.f;
    for (int c = 0; c < a.dqk; ++c) d = fmaf(qsh[qi * a.dqk + c], kr[c], d);
    tot += __builtin_amdgcn_exp2f(d * a.scale_log2 - qsh[nq * a.dqk + qi]);
  }
  a.scores[(int64_t)r * a.score_stride + s] = tot;
}

}  // namespace

hipError_t launch_attn_score(const ScoreArgs& a, hipStream_t s) {
  if (a.rows.n_rows == 0 || a.n_slots == 0) return hipSuccess;
  if (a.dtype == 0) {
    dim3 grid((a.n_slots + 255) / 256, a.rows.n_rows);
    const size_t lds = sizeof(float) * (size_t)a.n_qsets * a.hq * (a.dqk + 1);
    hipLaunchKernelGGL(attn_score_f32, grid, dim3(256), lds, s, a);
    return hipGetLastError();
  }
  // waves = hkv * sub = 8; each wave scores gpw groups of 64 entries;
  // enough workgroups to cover the chip several times
  const int sub = kScoreWaves / a.hkv;
  const int per_wg1 = 64 * sub;
  const int64_t wgs1 = (int64_t)((a.n_slots + per_wg1 - 1) / per_wg1) * a.rows.n_rows;
  int gpw = 1;
  while (gpw < 8 && wgs1 / (2 * gpw) >= 2048) gpw *= 2;
  const int per_wg = per_wg1 * gpw;
  dim3 grid((a.n_slots + per_wg - 1) / per_wg, a.rows.n_rows);
  dim3 block(64 * kScoreWaves);
  if (a.dqk == 128)
    hipLaunchKernelGGL(attn_score_mfma<128>, grid, block, 0, s, a, gpw, sub);
  else
    hipLaunchKernelGGL(attn_score_mfma<64>, grid, block, 0, s, a, gpw, sub);
  return hipGetLastError();
}

}  // namespace sa
