/*
 * oracle.c -- plain, slow, fp64 CPU oracle for indexer-driven top-k sparse
 * attention with index reuse.
 *
 * TEST INFRASTRUCTURE ONLY. The GPU library never loads, links or calls this
 * file; only the test suite, the package smoke check and the benchmark's
 * CPU-baseline leg do. It shares no code, header, table or helper with the HIP
 * path.
 *
 * Every function follows the plain definition of what it computes:
 *
 *  - Indexer score: the lightning-indexer equation of "Lecture 10 - Hybrid
 *    LLMs" (cs349d lecture page, section 5.1): the score of history entry s for
 *    query t is the sum over index heads j of w[t,j] * ReLU(q[t,j] . k[s]); the
 *    index key k[s] is one vector shared by all index heads.
 *  - Window + top-k: "HySparse2" page, section 7.2: the most recent w
 *    positions are always taken; at most k further positions are taken from
 *    outside that window, highest score first; nothing is counted twice.
 *    Ties are broken by the lower position.
 *  - Block-max candidate pool: "CSA, HCA and CSA2" page, section 3.2 (the
 *    Hierarchical Sparse Indexer): one set of scores gives every aligned block
 *    of positions its maximum; at most max_blocks blocks are kept; the pool is
 *    the union of their positions.
 *  - Joint softmax: "HySparse2" page, section 7.2: window and selected
 *    positions share one softmax normalisation and are read from one KV cache.
 *  - Full-attention selection score: "HySparse2" page, appendix A.1 (the FA
 *    layer selects by its own attention scores) and "Lecture 10", section 5.2
 *    (the per-position target sums the main attention over heads).
 *  - Storage formats: bfloat16; OCP FP8 E4M3 ("e4m3fn": bias 7, subnormals,
 *    no infinities, S.1111.111 is NaN, max 448); FP4 E2M1 (bias 1, values
 *    0, 0.5, 1, 1.5, 2, 3, 4, 6) with one E4M3 scale per 16 channels ("CSA, HCA
 *    and CSA2" page, section 3.2, the KV bytes and FP4 paragraph).
 *
 * All arithmetic is in double precision, in the order the definitions state
 * (channel sum ascending, then head sum ascending). Inputs are decoded exactly
 * from their storage format to double before use.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_E4M3 = 2, ORC_E2M1 = 3 };
enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_ENOMEM = -2 };

/* ------------------------------------------------------------------------ */
/* Storage decoding.                                                        */
/* ------------------------------------------------------------------------ */

/* bfloat16: the upper 16 bits of an IEEE-754 binary32. */
double orc_decode_bf16(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP FP8 E4M3 (e4m3fn): sign, 4 exponent bits (bias 7), 3 mantissa bits. */
double orc_decode_e4m3(uint8_t b) {
  int sign = (b >> 7) & 1;
  int e = (b >> 3) & 15;
  int m = b & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);          /* subnormal */
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);  /* normal */
  return sign ? -mag : mag;
}

/* FP4 E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit. */
double orc_decode_e2m1(uint8_t nibble) {
  int sign = (nibble >> 3) & 1;
  int e = (nibble >> 1) & 3;
  int m = nibble & 1;
  double mag;
  if (e == 0)
    mag = 0.5 * (double)m;                      /* subnormal: 0 or 0.5 */
  else
    mag = ldexp(1.0 + 0.5 * (double)m, e - 1);
  return sign ? -mag : mag;
}

static double load_elem(const void* base, int dtype, int64_t i) {
  switch (dtype) {
    case ORC_F32: return (double)((const float*)base)[i];
    case ORC_BF16: return orc_decode_bf16(((const uint16_t*)base)[i]);
    case ORC_E4M3: return orc_decode_e4m3(((const uint8_t*)base)[i]);
    default: return NAN;
  }
}

/* Channel c of an FP4 row: codes hold two channels per byte (even channel in
 * the low nibble); scales hold one E4M3 byte per 16 channels. */
static double load_fp4(const uint8_t* codes, const uint8_t* scales, int64_t c) {
  uint8_t byte = codes[c / 2];
  uint8_t nib = (c % 2 == 0) ? (byte & 15) : (byte >> 4);
  return orc_decode_e2m1(nib) * orc_decode_e4m3(scales[c / 16]);
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Domain of a query row.                                                   */
/* ------------------------------------------------------------------------ */

/* Number of cache entries visible to row r: an entry covers `stride` tokens
 * and is visible only when every one of its tokens is visible, i.e. entry e is
 * in the domain iff stride*(e+1) <= min(t+1, seq_len).  With stride 1 this is
 * the causal set {0..t} cut at the sequence length ("CSA, HCA and CSA2" page,
 * section 2.2: a query never reads an entry that contains a future token).
 * Padding rows (negative sequence or position) see nothing. */
static int64_t n_avail(int r, const int32_t* seq_of_row, const int32_t* pos_of_row,
                       const int32_t* seq_len, int stride) {
  int b = seq_of_row[r];
  int t = pos_of_row[r];
  if (b < 0 || t < 0) return 0;
  int64_t vis = (int64_t)t + 1;
  if (vis > seq_len[b]) vis = seq_len[b];
  if (vis < 0) vis = 0;
  return vis / stride;
}

int64_t orc_n_avail(int r, const int32_t* seq_of_row, const int32_t* pos_of_row,
                    const int32_t* seq_len, int stride) {
  return n_avail(r, seq_of_row, pos_of_row, seq_len, stride);
}

/* ------------------------------------------------------------------------ */
/* Indexer score.                                                           */
/* ------------------------------------------------------------------------ */

/*
 * q      [R][H][D] (q_dtype)         w [R][H] float
 * kidx   [B][Lcap][D] (k_dtype)      logical entry order, no paging
 * cand   optional [R][P]: score only positions cand[r][j], j < cand_count[r]
 * out    [R][out_stride] double: full mode writes out[r][s] for s < n_avail,
 *        candidate mode writes out[r][j] for j < cand_count[r]; every other
 *        slot of the row is set to NaN.
 */
int orc_index_score(int R, const int32_t* seq_of_row, const int32_t* pos_of_row,
                    const int32_t* seq_len, int stride, int H, int D, int q_dtype,
                    const void* q, const float* w, int k_dtype, const void* kidx, int64_t Lcap,
                    const int32_t* cand, const int32_t* cand_count, int64_t P, double* out,
                    int64_t out_stride) {
  if (R < 0 || H <= 0 || D <= 0 || stride <= 0) return ORC_EINVAL;
  for (int r = 0; r < R; ++r) {
    if (n_avail(r, seq_of_row, pos_of_row, seq_len, stride) > Lcap) return ORC_EINVAL;
    if (cand && cand_count[r] > P) return ORC_EINVAL;
  }
  for (int64_t i = 0; i < (int64_t)R * out_stride; ++i) out[i] = NAN;

  int64_t total = (int64_t)R * (cand ? P : Lcap);
#pragma omp parallel for schedule(dynamic, 256)
  for (int64_t it = 0; it < total; ++it) {
    int r = (int)(it / (cand ? P : Lcap));
    int64_t j = it % (cand ? P : Lcap);
    int64_t na = n_avail(r, seq_of_row, pos_of_row, seq_len, stride);
    int64_t s;
    if (cand) {
      if (j >= cand_count[r]) continue;
      s = cand[(int64_t)r * P + j];
      if (s < 0 || s >= na) continue; /* not a visible entry: left as NaN */
    } else {
      if (j >= na) continue;
      s = j;
    }
    int b = seq_of_row[r];
    const int64_t krow = ((int64_t)b * Lcap + s) * D;
    double score = 0.0;
    for (int h = 0; h < H; ++h) {
      const int64_t qrow = ((int64_t)r * H + h) * D;
      double dot = 0.0;
      for (int c = 0; c < D; ++c)
        dot += load_elem(q, q_dtype, qrow + c) * load_elem(kidx, k_dtype, krow + c);
      double relu = dot > 0.0 ? dot : 0.0;
      score += (double)w[(int64_t)r * H + h] * relu;
    }
    out[(int64_t)r * out_stride + j] = score;
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Selection.                                                               */
/* ------------------------------------------------------------------------ */

typedef struct {
  double key;
  int64_t pos;
} scored_pos;

/* Order: higher score first; equal scores -> lower position first.  The
 * comparison is on doubles, so -0 and +0 compare equal. */
static int cmp_score_desc_pos_asc(const void* a, const void* b) {
  const scored_pos* x = (const scored_pos*)a;
  const scored_pos* y = (const scored_pos*)b;
  if (x->key > y->key) return -1;
  if (x->key < y->key) return 1;
  if (x->pos < y->pos) return -1;
  if (x->pos > y->pos) return 1;
  return 0;
}

static int cmp_i64_asc(const void* a, const void* b) {
  int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
  return (x > y) - (x < y);
}

/*
 * Token top-k outside the window, and/or the block-max pool.
 *
 * scores [R][S] double (as written by orc_index_score; S is the row stride).
 * In candidate mode (cand != NULL, row stride P) scores[r][j] belongs to
 * position cand[r][j].
 *
 * Token mode (k > 0): candidates are the domain positions outside the window
 * W_t = [max(0, n_avail - window), n_avail); the first min(k, |C_t|) under
 * (score desc, position asc) are written ascending to idx[r][0..count), and
 * idx[r][count..k) = -1.
 *
 * Pool mode (block > 0, full mode only): blocks j = floor(s / block) over the
 * candidates C_t = [0, win_lo) (the visible positions outside the window;
 * with window 0 the whole domain), beta_j = max score of the block's
 * candidates; the first min(max_blocks, n_blocks) blocks under (beta desc,
 * j asc) are kept and the ascending union of their candidates is written to
 * pool[r][0..pool_count), pool[r][pool_count..max_blocks*block) = -1.  The
 * pool is therefore also a block-level selection in the index format ("HySparse2"
 * page, appendix A.1: the first generation selects 16 blocks of 64 tokens
 * next to a 128-token window).
 */
int orc_topk_select(int R, const int32_t* seq_of_row, const int32_t* pos_of_row,
                    const int32_t* seq_len, int stride, int window, const double* scores,
                    int64_t S, const int32_t* cand, const int32_t* cand_count, int64_t P, int k,
                    int32_t* idx, int32_t* count, int block, int max_blocks, int32_t* pool,
                    int32_t* pool_count) {
  if (R < 0 || stride <= 0 || window < 0 || k < 0) return ORC_EINVAL;
  if (block > 0 && cand) return ORC_EINVAL;
  int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < R; ++r) {
    int64_t na = n_avail(r, seq_of_row, pos_of_row, seq_len, stride);
    int64_t win_lo = na - window > 0 ? na - window : 0; /* first window position */
    if (k > 0) {
      int64_t ncand_max = cand ? cand_count[r] : win_lo;
      scored_pos* c = (scored_pos*)malloc(sizeof(scored_pos) * (size_t)(ncand_max > 0 ? ncand_max : 1));
      if (!c) {
        err = ORC_ENOMEM;
        continue;
      }
      int64_t nc = 0;
      for (int64_t j = 0; j < ncand_max; ++j) {
        int64_t s = cand ? cand[(int64_t)r * P + j] : j;
        if (s < 0 || s >= win_lo) continue; /* padding, or inside the window */
        c[nc].key = scores[(int64_t)r * S + j];
        c[nc].pos = s;
        ++nc;
      }
      qsort(c, (size_t)nc, sizeof(scored_pos), cmp_score_desc_pos_asc);
      int64_t take = nc < k ? nc : k;
      int64_t* sel = (int64_t*)malloc(sizeof(int64_t) * (size_t)(take > 0 ? take : 1));
      for (int64_t i = 0; i < take; ++i) sel[i] = c[i].pos;
      qsort(sel, (size_t)take, sizeof(int64_t), cmp_i64_asc);
      for (int64_t i = 0; i < k; ++i) idx[(int64_t)r * k + i] = i < take ? (int32_t)sel[i] : -1;
      count[r] = (int32_t)take;
      free(sel);
      free(c);
    }
    if (block > 0) {
      int64_t nb = (win_lo + block - 1) / block;
      scored_pos* bl = (scored_pos*)malloc(sizeof(scored_pos) * (size_t)(nb > 0 ? nb : 1));
      for (int64_t j = 0; j < nb; ++j) {
        double m = -INFINITY;
        for (int64_t s = j * block; s < (j + 1) * block && s < win_lo; ++s) {
          double v = scores[(int64_t)r * S + s];
          if (v > m) m = v;
        }
        bl[j].key = m;
        bl[j].pos = j;
      }
      qsort(bl, (size_t)nb, sizeof(scored_pos), cmp_score_desc_pos_asc);
      int64_t keep = nb < max_blocks ? nb : max_blocks;
      int64_t* kb = (int64_t*)malloc(sizeof(int64_t) * (size_t)(keep > 0 ? keep : 1));
      for (int64_t i = 0; i < keep; ++i) kb[i] = bl[i].pos;
      qsort(kb, (size_t)keep, sizeof(int64_t), cmp_i64_asc);
      int64_t cap = (int64_t)max_blocks * block, n = 0;
      for (int64_t i = 0; i < keep; ++i)
        for (int64_t s = kb[i] * block; s < (kb[i] + 1) * block && s < win_lo; ++s)
          pool[(int64_t)r * cap + n++] = (int32_t)s;
      pool_count[r] = (int32_t)n;
      for (; n < cap; ++n) pool[(int64_t)r * cap + n] = -1;
      free(kb);
      free(bl);
    }
  }
  return err;
}

/* ------------------------------------------------------------------------ */
/* Joint softmax attention over window + selected positions.                */
/* ------------------------------------------------------------------------ */

/*
 * q      [n_sets][R][Hq][dqk] (q_dtype)
 * K      [B][Lcap][Hkv][dqk]  (kv_dtype; for E2M1: bytes [B][Lcap][Hkv][dqk/2]
 *        with scales k_scale [B][Lcap][Hkv][dqk/16])
 * V      [B][Lcap][Hkv][dv], or, when v_from_k, the first dv channels of K
 * idx    [R][idx_stride] selected positions, count[r] of them (may be NULL
 *        for a window-only call)
 * o      [n_sets][R][Hq][dv] double, lse [n_sets][R][Hq] double (natural log)
 *
 * Access set A_t = W_t U T_t with W_t = [max(0, n_avail - window), n_avail)
 * and T_t = {idx[r][i] : i < count[r]}; a position is counted once. Query
 * head h reads KV head floor(h * Hkv / Hq). logit_s = scale * q . K_s; one
 * softmax over A_t; o = sum p_s V_s; lse = log sum exp(logit). Empty A_t gives
 * o = 0 and lse = -inf.
 *
 * Optional per-head sink bias and output sigmoid gate ("HySparse2" page,
 * section 17.1: every SA layer has an output sigmoid gate and a learnable
 * per-head sink bias): sink [n_sets][Hq] (float, may be NULL) is the logit of
 * one more entry whose value row is zero, so it joins the normaliser only:
 * p_s = exp(logit_s) / (exp(sink) + sum exp(logit)), lse = log(exp(sink) +
 * sum exp(logit)), and an empty A_t gives o = 0, lse = sink.  gate
 * [n_sets][R][Hq][dv] (gate_dtype, may be NULL) multiplies output channel c by
 * 1 / (1 + exp(-gate[c])).
 */
int orc_attention(int n_sets, int R, const int32_t* seq_of_row, const int32_t* pos_of_row,
                  const int32_t* seq_len, int stride, int window, int Hq, int Hkv, int dqk,
                  int dv, int q_dtype, const void* q, int kv_dtype, const void* K,
                  const uint8_t* k_scale, const void* V, const uint8_t* v_scale, int v_from_k,
                  int64_t Lcap, const int32_t* idx, int64_t idx_stride, const int32_t* count,
                  float scale, const float* sink, int gate_dtype, const void* gate, double* o,
                  double* lse) {
  if (n_sets <= 0 || R < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || dqk <= 0 || dv <= 0)
    return ORC_EINVAL;
  if (v_from_k && dv > dqk) return ORC_EINVAL;
  if (kv_dtype == ORC_E2M1 && (dqk % 16 != 0 || dv % 16 != 0)) return ORC_EINVAL;
  const double sc = (double)scale;
  int64_t total = (int64_t)n_sets * R * Hq;
  int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t it = 0; it < total; ++it) {
    int h = (int)(it % Hq);
    int r = (int)((it / Hq) % R);
    int set = (int)(it / ((int64_t)Hq * R));
    int64_t na = n_avail(r, seq_of_row, pos_of_row, seq_len, stride);
    int64_t win_lo = na - window > 0 ? na - window : 0;
    int g = (int)((int64_t)h * Hkv / Hq);
    int b = seq_of_row[r];
    double* orow = o + it * dv;
    for (int c = 0; c < dv; ++c) orow[c] = 0.0;

    /* Gather the access set (window, then selected positions), without
     * duplicates, then sort it so the position order is canonical. */
    int64_t nsel = count ? count[r] : 0;
    int64_t cap = (na - win_lo) + nsel;
    int64_t* A = (int64_t*)malloc(sizeof(int64_t) * (size_t)(cap > 0 ? cap : 1));
    double* logit = (double*)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
    if (!A || !logit) {
      err = ORC_ENOMEM;
      free(A);
      free(logit);
      continue;
    }
    int64_t n = 0;
    for (int64_t s = win_lo; s < na; ++s) A[n++] = s;
    for (int64_t i = 0; i < nsel; ++i) {
      int64_t s = idx[(int64_t)r * idx_stride + i];
      if (s < 0) continue;
      if (s >= Lcap) {
        err = ORC_EINVAL;
        continue;
      }
      A[n++] = s;
    }
    qsort(A, (size_t)n, sizeof(int64_t), cmp_i64_asc);
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i)
      if (m == 0 || A[i] != A[m - 1]) A[m++] = A[i];
    n = m;

    const double sk = sink ? (double)sink[(int64_t)set * Hq + h] : -INFINITY;
    if (n == 0 || b < 0) {
      lse[it] = sk;
      free(A);
      free(logit);
      continue;
    }
    const int64_t qrow = (((int64_t)set * R + r) * Hq + h) * dqk;
    double mx = -INFINITY;
    for (int64_t i = 0; i < n; ++i) {
      int64_t row = ((int64_t)b * Lcap + A[i]) * Hkv + g;
      double dot = 0.0;
      for (int c = 0; c < dqk; ++c) {
        double kv;
        if (kv_dtype == ORC_E2M1)
          kv = load_fp4((const uint8_t*)K + row * (dqk / 2), k_scale + row * (dqk / 16), c);
        else
          kv = load_elem(K, kv_dtype, row * dqk + c);
        dot += load_elem(q, q_dtype, qrow + c) * kv;
      }
      logit[i] = sc * dot;
      if (logit[i] > mx) mx = logit[i];
    }
    if (sk > mx) mx = sk;
    double sum = sink ? exp(sk - mx) : 0.0;
    for (int64_t i = 0; i < n; ++i) sum += exp(logit[i] - mx);
    for (int64_t i = 0; i < n; ++i) {
      double p = exp(logit[i] - mx) / sum;
      int64_t row = ((int64_t)b * Lcap + A[i]) * Hkv + g;
      for (int c = 0; c < dv; ++c) {
        double vv;
        if (v_from_k) {
          if (kv_dtype == ORC_E2M1)
            vv = load_fp4((const uint8_t*)K + row * (dqk / 2), k_scale + row * (dqk / 16), c);
          else
            vv = load_elem(K, kv_dtype, row * dqk + c);
        } else {
          if (kv_dtype == ORC_E2M1)
            vv = load_fp4((const uint8_t*)V + row * (dv / 2), v_scale + row * (dv / 16), c);
          else
            vv = load_elem(V, kv_dtype, row * dv + c);
        }
        orow[c] += p * vv;
      }
    }
    lse[it] = mx + log(sum);
    if (gate)
      for (int c = 0; c < dv; ++c)
        orow[c] *= 1.0 / (1.0 + exp(-load_elem(gate, gate_dtype, it * dv + c)));
    free(A);
    free(logit);
  }
  return err;
}

/* ------------------------------------------------------------------------ */
/* Full-attention selection score.                                          */
/* ------------------------------------------------------------------------ */

/*
 * The selection signal of a full-attention layer ("HySparse2" page, appendix
 * A.1: the FA layer computes ordinary full attention and picks the important
 * history positions from those attention scores, which its SA layers then
 * reuse; "Lecture 10 - Hybrid LLMs", section 5.2: the per-position target is
 * the main attention's scores summed over heads):
 *
 *   score[r][s] = sum over query sets i and query heads h of p_{i,h}(s),
 *   p_{i,h} = softmax over the row's whole visible domain of
 *             scale * q[i][r][h] . K[s][g(h)],  g(h) = floor(h * Hkv / Hq).
 *
 * q [n_sets][R][Hq][dqk]; K logical [B][Lcap][Hkv][dqk].  out [R][out_stride]:
 * out[r][s] for s < n_avail, NaN elsewhere (and for padding rows).
 */
int orc_fa_score(int n_sets, int R, const int32_t* seq_of_row, const int32_t* pos_of_row,
                 const int32_t* seq_len, int stride, int Hq, int Hkv, int dqk, int q_dtype,
                 const void* q, int kv_dtype, const void* K, int64_t Lcap, float scale,
                 double* out, int64_t out_stride) {
  if (n_sets <= 0 || R < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || dqk <= 0 || stride <= 0)
    return ORC_EINVAL;
  if (kv_dtype == ORC_E2M1) return ORC_EINVAL;
  for (int r = 0; r < R; ++r)
    if (n_avail(r, seq_of_row, pos_of_row, seq_len, stride) > Lcap) return ORC_EINVAL;
  for (int64_t i = 0; i < (int64_t)R * out_stride; ++i) out[i] = NAN;
  const double sc = (double)scale;
  int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < R; ++r) {
    int64_t na = n_avail(r, seq_of_row, pos_of_row, seq_len, stride);
    int b = seq_of_row[r];
    if (na == 0 || b < 0) continue;
    double* acc = (double*)calloc((size_t)na, sizeof(double));
    double* logit = (double*)malloc(sizeof(double) * (size_t)na);
    if (!acc || !logit) {
      err = ORC_ENOMEM;
      free(acc);
      free(logit);
      continue;
    }
    for (int set = 0; set < n_sets; ++set) {
      for (int h = 0; h < Hq; ++h) {
        int g = (int)((int64_t)h * Hkv / Hq);
        const int64_t qrow = (((int64_t)set * R + r) * Hq + h) * dqk;
        double mx = -INFINITY;
        for (int64_t s = 0; s < na; ++s) {
          int64_t row = ((int64_t)b * Lcap + s) * Hkv + g;
          double dot = 0.0;
          for (int c = 0; c < dqk; ++c)
            dot += load_elem(q, q_dtype, qrow + c) * load_elem(K, kv_dtype, row * dqk + c);
          logit[s] = sc * dot;
          if (logit[s] > mx) mx = logit[s];
        }
        double sum = 0.0;
        for (int64_t s = 0; s < na; ++s) sum += exp(logit[s] - mx);
        for (int64_t s = 0; s < na; ++s) acc[s] += exp(logit[s] - mx) / sum;
      }
    }
    for (int64_t s = 0; s < na; ++s) out[(int64_t)r * out_stride + s] = acc[s];
    free(acc);
    free(logit);
  }
  return err;
}
