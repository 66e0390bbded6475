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
// head and query set.  Per 32-entry tile:
//   1. the workgroup gathers the 32 K (and V) rows through the block table
//      into LDS (FP4 rows are dequantised exactly to bf16 on the way);
//   2. each wave computes S^T = K . Q^T for its 16 query rows with
//      v_mfma_f32_16x16x32_bf16 (entries on M, query rows on N), so each lane
//      ends up holding 8 logits of ONE query row;
//   3. online softmax in fp32 (exp2 domain), per query row;
//   4. O^T += V^T . P^T with the contraction order permuted so that the
//      lane's 8 probabilities are directly its B operand; the V^T operand is
//      built from 16-byte LDS reads by an in-register 8x8 bf16 transpose
//      (v_perm).  O^T keeps each lane on one query row, so the online-softmax
//      rescale and the final normalisation need no cross-lane traffic;
//      row statistics are reduced with the gfx950 lane-swap instructions.
// Long entry lists are split across workgroups; a combine kernel merges the
// (max, sum, unnormalised O) partials.  F32 inputs use a plain VALU kernel.
#include "kernels.hpp"

namespace sa {

namespace {

constexpr int kTile = 32;   // entries per tile

enum { KV_SEPARATE = 0, KV_SHARED = 1, KV_FP4 = 2 };

__device__ __forceinline__ uint32_t lo16x2(uint32_t a, uint32_t b) {
  return (a & 0xFFFFu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi16x2(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xFFFF0000u);
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

constexpr int kNW = 4;           // waves per workgroup (one per SIMD)
constexpr int kMaxEntries = 2048;  // entries per workgroup (slot table size)

template <int DQK, int DV, int KV>
struct AttnLds {
  static constexpr int KROW = DQK + 8;  // bf16 elements per LDS row (padded)
  static constexpr int VROW = DV + 8;
  static constexpr bool HAS_V = KV == KV_SEPARATE;
  uint16_t k[2][kTile * KROW];
  uint16_t v[2][HAS_V ? kTile * VROW : 1];
  int32_t slot[kMaxEntries + 8 * kTile];  // cache slot of every entry (-1: none)
};

// Per-thread share of one tile of gathered rows, held in registers between
// the global load and the LDS store (the prefetch ring).
template <int DQK, int DV, int KV>
struct TileRegs {
  static constexpr bool FP4 = KV == KV_FP4;
  static constexpr int CPR_K = FP4 ? DQK / 32 : DQK / 8;  // 16-byte chunks per K row
  static constexpr int CPR_V = KV == KV_SEPARATE ? DV / 8 : 0;
  static constexpr int C_K = kTile * CPR_K;
  static constexpr int C_ALL = C_K + kTile * CPR_V;
  static constexpr int U = (C_ALL + 64 * kNW - 1) / (64 * kNW);
  u32x4 v[U];
  uint32_t sc[FP4 ? U : 1];  // FP4: the two E4M3 scales of each 32-channel chunk
};

template <int DQK, int DV, int KV, int D>
__global__ __launch_bounds__(64 * kNW, 1) void attn_mfma(AttnArgs a, int per_split) {
  using L = AttnLds<DQK, DV, KV>;
  using T = TileRegs<DQK, DV, KV>;
  __shared__ __align__(16) L lds;
  constexpr int KS = DQK / 32;   // k-steps of the S MFMA
  constexpr int QV = DQK / 32;   // 16-byte q vectors per lane
  constexpr int NJB = DV / 128;  // 128-channel blocks of V
  constexpr int NT = DV / 16;    // N tiles of O
  constexpr int NTH = 64 * kNW;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, gq = lane >> 4;
  const int sp = blockIdx.x;
  const int r = blockIdx.y / a.hkv, g = blockIdx.y % a.hkv;
  const int G = a.hq / a.hkv;
  const int Mq = a.n_qsets * G;
  const int qrow0 = (blockIdx.z * kNW + wave) * 16;
  const bool active = qrow0 < Mq;

  const RowInfo ri = row_info(a.rows, r);
  const int n_w = ri.n_avail - ri.win_lo;
  const int cnt = (a.idx && ri.b >= 0) ? a.count[r] : 0;
  const int n_e = ri.b < 0 ? 0 : n_w + cnt;
  const int e0 = sp * per_split, e1 = min(n_e, e0 + per_split);
  const int ne = max(0, e1 - e0);
  const int ntiles = (ne + kTile - 1) / kTile;
  const int32_t* idx = a.idx ? a.idx + (int64_t)r * a.idx_stride : nullptr;

  // Cache slot of every entry of this range, once: the window entries, then
  // the selected ones, through the block table.  Padding to whole tiles, and
  // the D tiles past the end that the prefetch ring reads, are -1.
  for (int i = tid; i < (ntiles + D) * kTile; i += NTH) {
    int slot = -1;
    if (i < ne) {
      const int e = e0 + i;
      const int pos = e < n_w ? ri.win_lo + e : idx[e - n_w];
      if (pos >= 0) slot = (int)cache_slot(a.k, ri.b, pos);
    }
    lds.slot[i] = slot;
  }

  // Query rows of this wave as the B operand (query row = col).
  u32x4 qv[QV];
  {
    const int qr = qrow0 + col;
    if (active && qr < Mq) {
      const int set = qr / G, h = g * G + qr % G;
      const u32x4* qp = reinterpret_cast<const u32x4*>(
          reinterpret_cast<const uint16_t*>(a.q) +
          (((int64_t)set * a.rows.n_rows + r) * a.hq + h) * DQK + gq * (DQK / 4));
#pragma unroll
      for (int i = 0; i < QV; ++i) qv[i] = qp[i];
    } else {
#pragma unroll
      for (int i = 0; i < QV; ++i) qv[i] = u32x4{0, 0, 0, 0};
    }
  }
  __syncthreads();

  // Issue the global loads of tile t into registers.  Branch-free, so the
  // compiler can keep D tiles of loads in flight: an entry without a slot
  // reads slot 0 (always backed by the cache) and is zeroed at store time.
  auto load_tile = [&](int t, T& regs) {
#pragma unroll
    for (int u = 0; u < T::U; ++u) {
      int c = tid + NTH * u;
      if (T::C_ALL % NTH != 0) c = min(c, T::C_ALL - 1);
      const bool is_k = c < T::C_K;
      const int cc = is_k ? c : c - T::C_K;
      const int cpr = is_k ? T::CPR_K : T::CPR_V;
      const int e = cc / cpr, part = cc % cpr;
      const int64_t slot = max(lds.slot[t * kTile + e], 0);
      if constexpr (T::FP4) {
        regs.v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
            a.k.data + slot * a.k.row_stride + g * (DQK / 2) + part * 16));
        regs.sc[u] = *reinterpret_cast<const uint16_t*>(a.k.scale + slot * a.k.scale_stride +
                                                        g * (DQK / 16) + part * 2);
      } else {
        const char* base = is_k ? a.k.data + slot * a.k.row_stride + g * (DQK * 2)
                                : a.v.data + slot * a.v.row_stride + g * (DV * 2);
        regs.v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + part * 16));
      }
    }
  };
  // Store tile t's registers into LDS buffer `buf` (FP4 is dequantised here);
  // rows of entries without a slot become zeros.
  auto store_tile = [&](const T& regs, int buf, int t) {
#pragma unroll
    for (int u = 0; u < T::U; ++u) {
      const int c = tid + NTH * u;
      if (T::C_ALL % NTH != 0 && c >= T::C_ALL) continue;
      if constexpr (T::FP4) {
        const int e = c / T::CPR_K, part = c % T::CPR_K;
        const bool ok = lds.slot[t * kTile + e] >= 0;
        uint32_t vals[16];
        fp4_dequant32(regs.v[u], regs.sc[u] & 0xFFu, regs.sc[u] >> 8, vals);
        u32x4* dst = reinterpret_cast<u32x4*>(&lds.k[buf][e * L::KROW + part * 32]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[i] = ok ? u32x4{vals[4 * i], vals[4 * i + 1], vals[4 * i + 2], vals[4 * i + 3]}
                      : u32x4{0, 0, 0, 0};
      } else if (c < T::C_K) {
        const int e = c / T::CPR_K, part = c % T::CPR_K;
        const bool ok = lds.slot[t * kTile + e] >= 0;
        *reinterpret_cast<u32x4*>(&lds.k[buf][e * L::KROW + part * 8]) =
            ok ? regs.v[u] : u32x4{0, 0, 0, 0};
      } else {
        const int cc = c - T::C_K;
        const int e = cc / T::CPR_V, part = cc % T::CPR_V;
        const bool ok = lds.slot[t * kTile + e] >= 0;
        *reinterpret_cast<u32x4*>(&lds.v[buf][e * L::VROW + part * 8]) =
            ok ? regs.v[u] : u32x4{0, 0, 0, 0};
      }
    }
  };

  f32x4 O[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_huge_valf(), l_run = 0.0f;

  auto compute = [&](int buf, int t) {
    const uint16_t* kb = lds.k[buf];
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
    const float m_new = fmaxf(m_run, tmax);
    float alpha = 1.0f;
    float psum = 0.0f;
    float p[2][4];
    if (m_new == -__builtin_huge_valf()) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[mt][i] = 0.0f;
    } else {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[mt][i] = exp2f(s[mt][i] - m_new);
          psum += p[mt][i];
        }
    }
    psum = xor16_32_sum(psum);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // O^T holds only this lane's query row (col): the rescale is lane-local
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) O[tt][i] *= alpha;

    // P^T as the B operand: k-slot 8*gq + i <-> entry (i<4 ? 4gq+i : 16+4gq+i-4)
    u32x4 pa;
    pa[0] = pack_bf16x2(p[0][0], p[0][1]);
    pa[1] = pack_bf16x2(p[0][2], p[0][3]);
    pa[2] = pack_bf16x2(p[1][0], p[1][1]);
    pa[3] = pack_bf16x2(p[1][2], p[1][3]);
    const bf16x8 pab = __builtin_bit_cast(bf16x8, pa);
    const uint16_t* vbase = KV == KV_SEPARATE ? lds.v[buf] : kb;
    constexpr int VR = KV == KV_SEPARATE ? L::VROW : L::KROW;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
      // V^T as the A operand: lane col takes channels 128jb + 8col + j of the
      // 8 entries of its k-slots (an 8x8 bf16 transpose in registers), so
      // M-tile 8jb + j row m is channel 128jb + 8m + j.
      u32x4 R[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = i < 4 ? 4 * gq + i : 16 + 4 * gq + (i - 4);
        R[i] = *reinterpret_cast<const u32x4*>(vbase + e * VR + jb * 128 + col * 8);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u32x4 b;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          b[qd] = (j & 1) ? hi16x2(R[2 * qd][j >> 1], R[2 * qd + 1][j >> 1])
                          : lo16x2(R[2 * qd][j >> 1], R[2 * qd + 1][j >> 1]);
        O[jb * 8 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, b), pab, O[jb * 8 + j], 0, 0, 0);
      }
    }
  };

  // Prefetch ring: tile t's rows are loaded D tiles ahead of their use.  Full
  // groups of D tiles run without guards (D is even, so the LDS buffer of
  // each unrolled step is static); the last partial group is guarded.
  static_assert(D % 2 == 0, "prefetch depth must be even");
  T ring[D];
#pragma unroll
  for (int u = 0; u < D; ++u) load_tile(u, ring[u]);
  int t0 = 0;
  for (; t0 + D <= ntiles; t0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      store_tile(ring[u], u & 1, t0 + u);
      __syncthreads();
      load_tile(t0 + u + D, ring[u]);
      if (active) compute(u & 1, t0 + u);
    }
  }
#pragma unroll
  for (int u = 0; u < D; ++u) {
    if (t0 + u < ntiles) {
      store_tile(ring[u], u & 1, t0 + u);
      __syncthreads();
      if (active) compute(u & 1, t0 + u);
    }
  }

  if (!active) return;
  // Output: lane holds O^T for query row qrow0 + col: O[8jb + j][i] is channel
  // 128jb + 8(4gq + i) + j, so each (jb, i) is 8 contiguous channels.
  const int qr = qrow0 + col;
  if (qr >= Mq) return;
  const int R = a.rows.n_rows;
  const int set = qr / G, h = g * G + qr % G;
  const int64_t orow = ((int64_t)set * R + r) * a.hq + h;
  if (a.n_split == 1) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c0 = jb * 128 + 32 * gq + 8 * i;
        if (a.o_dtype == 1) {
          u32x4 pk;
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            pk[qd] = pack_bf16x2(O[jb * 8 + 2 * qd][i] * inv, O[jb * 8 + 2 * qd + 1][i] * inv);
          *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.o) + orow * DV + c0) = pk;
        } else {
          float* op = reinterpret_cast<float*>(a.o) + orow * DV + c0;
          f32x4 v0 = {O[jb * 8 + 0][i] * inv, O[jb * 8 + 1][i] * inv, O[jb * 8 + 2][i] * inv,
                      O[jb * 8 + 3][i] * inv};
          f32x4 v1 = {O[jb * 8 + 4][i] * inv, O[jb * 8 + 5][i] * inv, O[jb * 8 + 6][i] * inv,
                      O[jb * 8 + 7][i] * inv};
          reinterpret_cast<f32x4*>(op)[0] = v0;
          reinterpret_cast<f32x4*>(op)[1] = v1;
        }
      }
    if (a.lse && gq == 0)
      a.lse[orow] = l_run > 0.0f ? (m_run + __log2f(l_run)) * 0.6931471805599453f
                                 : -__builtin_huge_valf();
  } else {
    const int64_t nrows = (int64_t)a.n_qsets * R * a.hq;
    float* po = a.part + ((int64_t)sp * nrows + orow) * DV;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float* op = po + jb * 128 + 32 * gq + 8 * i;
        f32x4 v0 = {O[jb * 8 + 0][i], O[jb * 8 + 1][i], O[jb * 8 + 2][i], O[jb * 8 + 3][i]};
        f32x4 v1 = {O[jb * 8 + 4][i], O[jb * 8 + 5][i], O[jb * 8 + 6][i], O[jb * 8 + 7][i]};
        reinterpret_cast<f32x4*>(op)[0] = v0;
        reinterpret_cast<f32x4*>(op)[1] = v1;
      }
    if (gq == 0) {
      float* ml = a.part + (int64_t)a.n_split * nrows * DV + ((int64_t)sp * nrows + orow) * 2;
      ml[0] = m_run;
      ml[1] = l_run;
    }
  }
}

// Merge split partials: o = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i.
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nrows = (int64_t)a.n_qsets * a.rows.n_rows * a.hq;
  if (row >= nrows) return;
  const int DV = a.dv;
  const float* ml = a.part + (int64_t)a.n_split * nrows * DV;
  float M = -__builtin_huge_valf();
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, ml[((int64_t)s * nrows + row) * 2]);
  float Lsum = 0.0f;
  for (int s = 0; s < a.n_split; ++s) {
    const float m = ml[((int64_t)s * nrows + row) * 2], l = ml[((int64_t)s * nrows + row) * 2 + 1];
    if (l > 0.0f) Lsum += exp2f(m - M) * l;
  }
  const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  for (int c = lane; c < DV; c += 64) {
    float acc = 0.0f;
    for (int s = 0; s < a.n_split; ++s) {
      const float m = ml[((int64_t)s * nrows + row) * 2], l = ml[((int64_t)s * nrows + row) * 2 + 1];
      if (l > 0.0f) acc += exp2f(m - M) * a.part[((int64_t)s * nrows + row) * DV + c];
    }
    acc *= inv;
    if (a.o_dtype == 1)
      reinterpret_cast<uint16_t*>(a.o)[row * DV + c] = (uint16_t)f32_to_bf16_bits(acc);
    else
      reinterpret_cast<float*>(a.o)[row * DV + c] = acc;
  }
  if (a.lse && lane == 0)
    a.lse[row] = Lsum > 0.0f ? (M + __log2f(Lsum)) * 0.6931471805599453f : -__builtin_huge_valf();
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
  const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  for (int k = 0; k < 4; ++k) {
    const int c = lane + 64 * k;
    if (c >= a.dv) continue;
    if (a.o_dtype == 1)
      reinterpret_cast<uint16_t*>(a.o)[orow * a.dv + c] = (uint16_t)f32_to_bf16_bits(acc[k] * inv);
    else
      reinterpret_cast<float*>(a.o)[orow * a.dv + c] = acc[k] * inv;
  }
  if (a.lse && lane == 0)
    a.lse[orow] = l_run > 0.0f ? (m_run + __log2f(l_run)) * 0.6931471805599453f
                               : -__builtin_huge_valf();
}

template <int DQK, int DV, int KV, int D>
hipError_t launch_mfma_attn(const AttnArgs& a, hipStream_t s) {
  const int G = a.hq / a.hkv;
  const int tiles = (a.n_qsets * G + 15) / 16;
  const int groups = (tiles + kNW - 1) / kNW;
  const int per = ((a.max_entries + a.n_split - 1) / a.n_split + kTile - 1) / kTile * kTile;
  dim3 grid(a.n_split, a.rows.n_rows * a.hkv, groups);
  hipLaunchKernelGGL((attn_mfma<DQK, DV, KV, D>), grid, dim3(64 * kNW), 0, s, a, per);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  const int64_t nrows = (int64_t)a.n_qsets * a.rows.n_rows * a.hq;
  hipLaunchKernelGGL(attn_combine, dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// Splits per row so that the grid covers the chip about twice; never below
// one 32-entry tile per split.
void attn_plan(AttnArgs& a) {
  a.n_split = 1;
  if (a.dtype == 0) return;
  const int G = a.hq / a.hkv;
  const int tiles = (a.n_qsets * G + 15) / 16;
  const int64_t base = (int64_t)a.rows.n_rows * a.hkv * ((tiles + kNW - 1) / kNW);
  const int max_split = (a.max_entries + kTile - 1) / kTile;
  // enough entry ranges to occupy the chip, each within the slot table
  int ns = (a.max_entries + kMaxEntries - 1) / kMaxEntries;
  // wide value rows make split partials expensive: stop earlier
  const int cap = a.dv >= 512 ? 4 : max_split;
  while (ns < max_split && ns < cap && base * ns < 256) ++ns;
  a.n_split = ns < 1 ? 1 : ns;
}

size_t attn_workspace_bytes(const AttnArgs& a) {
  if (a.n_split <= 1) return 0;
  const int64_t nrows = (int64_t)a.n_qsets * a.rows.n_rows * a.hq;
  return (size_t)a.n_split * nrows * (a.dv + 2) * sizeof(float);
}

hipError_t launch_attn_gather(const AttnArgs& a, hipStream_t s) {
  if (a.rows.n_rows == 0) return hipSuccess;
  if (a.dtype == 0) {
    const int G = a.hq / a.hkv;
    dim3 grid(a.rows.n_rows * a.hkv, (a.n_qsets * G + 3) / 4);
    hipLaunchKernelGGL(attn_f32, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (a.kv_kind == KV_SEPARATE) {
    if (a.dqk == 128 && a.dv == 128) return launch_mfma_attn<128, 128, KV_SEPARATE, 4>(a, s);
    if (a.dqk == 256 && a.dv == 256) return launch_mfma_attn<256, 256, KV_SEPARATE, 2>(a, s);
  } else if (a.kv_kind == KV_SHARED) {
    if (a.dqk == 576 && a.dv == 512) return launch_mfma_attn<576, 512, KV_SHARED, 2>(a, s);
    if (a.dqk == 512 && a.dv == 512) return launch_mfma_attn<512, 512, KV_SHARED, 2>(a, s);
    if (a.dqk == 128 && a.dv == 128) return launch_mfma_attn<128, 128, KV_SHARED, 4>(a, s);
  } else if (a.kv_kind == KV_FP4) {
    if (a.dqk == 512 && a.dv == 512) return launch_mfma_attn<512, 512, KV_FP4, 4>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
