// Device-side helpers shared by the gfx950 kernels of the sparse-attention
// library: the row domain, paged-cache addressing, number formats, orderable
// score keys and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr float kLog2e = 1.4426950408889634f;

// The query rows of a call.  Entry e of sequence b is visible to a row at
// token position t iff stride*(e+1) <= min(t+1, seq_len[b]).
struct RowsDev {
  const int32_t* seq_of_row;
  const int32_t* pos_of_row;
  const int32_t* seq_len;
  int32_t n_rows;
  int32_t stride;
  int32_t window;
};

struct RowInfo {
  int32_t b;        // sequence, or -1 for a padding row
  int32_t n_avail;  // visible entries [0, n_avail)
  int32_t win_lo;   // first window entry; candidates are [0, win_lo)
};

__device__ __forceinline__ RowInfo row_info(const RowsDev& R, int r) {
  RowInfo ri;
  int b = R.seq_of_row[r];
  int t = R.pos_of_row[r];
  if (b < 0 || t < 0) {
    ri.b = -1;
    ri.n_avail = 0;
    ri.win_lo = 0;
    return ri;
  }
  int vis = min(t + 1, R.seq_len[b]);
  vis = max(vis, 0);
  ri.b = b;
  ri.n_avail = vis / R.stride;
  ri.win_lo = max(0, ri.n_avail - R.window);
  return ri;
}

// A paged cache of rows.  Entry e of sequence b lives at slot
// page*page_size + e%page_size where page = block_table[b][e/page_size]
// (identity map without a block table).
struct CacheDev {
  const char* data;
  const uint8_t* scale;
  const int32_t* block_table;
  int64_t row_stride;
  int64_t scale_stride;
  int32_t page_size;
  int32_t page_shift;  // log2(page_size), or -1 if not a power of two
  int32_t max_pages;
  int32_t pad;
};

__device__ __forceinline__ int64_t cache_slot(const CacheDev& c, int b, int e) {
  int pg, off;
  if (c.page_shift >= 0) {
    pg = e >> c.page_shift;
    off = e & (c.page_size - 1);
  } else {
    pg = e / c.page_size;
    off = e - pg * c.page_size;
  }
  int64_t lp = (int64_t)b * c.max_pages + pg;
  int64_t p = c.block_table ? (int64_t)c.block_table[lp] : lp;
  return p * c.page_size + off;
}

__device__ __forceinline__ const char* cache_row(const CacheDev& c, int b, int e) {
  return c.data + cache_slot(c, b, e) * c.row_stride;
}

// ---------------------------------------------------------------------------
// Number formats
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) {
  return __uint_as_float(h16 << 16);
}

// Round-to-nearest-even float -> bfloat16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats -> packed bfloat16 pair (lo in the low half), round to nearest
// even: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// OCP E4M3 (e4m3fn) byte -> float.  NaN codes are not expected in scales.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (b & 0x80u) ? -mag : mag;
}

// FP4 E2M1 nibble -> float.
__device__ __forceinline__ float e2m1_to_f32(uint32_t nib) {
  // magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 in units of 0.5
  const uint32_t halves = 0xC8643210u;  // nibble k holds 2*value of code k
  float mag = (float)((halves >> (4 * (nib & 7u))) & 15u) * 0.5f;
  return (nib & 8u) ? -mag : mag;
}

// max(x, 0) for a finite float in one v_max_i32: a negative float (and -0)
// is a negative int32, so the integer max with 0 gives +0, and a positive
// float keeps its bits.  (fmaxf also canonicalises its operand: two
// instructions.)
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// ---------------------------------------------------------------------------
// Orderable score keys: a larger float maps to a larger uint32; -0 maps to
// the key of +0 so the two tie.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float x) {
  // adding +0 turns -0 into +0 and keeps every other value (f32 denormals
  // are not flushed); then negatives flip all bits, the rest the sign bit
  const uint32_t u = __float_as_uint(x + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// ---------------------------------------------------------------------------
// Wave (64-lane) reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Butterfly reductions across the four 16-lane groups of a wave with the
// gfx950 lane-swap VALU instructions (no LDS round trip): after the two
// steps every lane holds the reduction over lanes {l, l^16, l^32, l^48}.
__device__ __forceinline__ float xor16_32_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xor16_32_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Transposed reduction of four per-lane values: afterwards lane group g
// (lanes 16g .. 16g+15) holds r_g summed over lanes {l, l^16, l^32, l^48}.
// The 32-lane swap pairs (r0, r2) and (r1, r3); the 16-lane swap then pairs
// the two half sums: three swaps and three adds for four reductions.
__device__ __forceinline__ float sum4_transposed(float r0, float r1, float r2, float r3) {
  const auto x02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(r0), __float_as_uint(r2), false, false);
  const auto x13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(r1), __float_as_uint(r3), false, false);
  const float h0 = __uint_as_float(x02[0]) + __uint_as_float(x02[1]);  // lanes < 32: r0, else r2
  const float h1 = __uint_as_float(x13[0]) + __uint_as_float(x13[1]);  // lanes < 32: r1, else r3
  const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(h0), __float_as_uint(h1), false, false);
  return __uint_as_float(y[0]) + __uint_as_float(y[1]);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

}  // namespace sa
