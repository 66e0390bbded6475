// C ABI of the sparse-attention library: host-side validation, workspace
// sizing and kernel dispatch.  Every entry point returns an sa_status and
// never throws; the message of the last failure on the calling thread is
// available from sa_last_error().
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "sparse_attn.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

sa_status fail(sa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

#define CHECK(cond, st, ...)              \
  do {                                    \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(int dtype) {
  switch (dtype) {
    case SA_F32: return 4;
    case SA_BF16: return 2;
    case SA_FP8_E4M3: return 1;
    default: return 0;
  }
}

sa_status check_rows(const sa_rows& r, const char* op) {
  CHECK(r.n_rows >= 0 && r.n_seqs >= 0, SA_ERR_SHAPE, "%s: negative n_rows or n_seqs", op);
  if (r.n_rows == 0) return SA_OK;
  CHECK(r.seq_of_row && r.pos_of_row && r.seq_len, SA_ERR_NULL,
        "%s: rows.seq_of_row, pos_of_row and seq_len are required", op);
  CHECK(r.stride >= 1, SA_ERR_SHAPE, "%s: rows.stride must be >= 1", op);
  CHECK(r.window >= 0, SA_ERR_SHAPE, "%s: rows.window must be >= 0", op);
  return SA_OK;
}

sa::RowsDev to_dev(const sa_rows& r) {
  sa::RowsDev d;
  d.seq_of_row = r.seq_of_row;
  d.pos_of_row = r.pos_of_row;
  d.seq_len = r.seq_len;
  d.n_rows = r.n_rows;
  d.stride = r.stride;
  d.window = r.window;
  return d;
}

sa_status check_cache(const sa_cache& c, const char* op, const char* name, int64_t min_row_bytes) {
  CHECK(c.data, SA_ERR_NULL, "%s: %s.data is NULL", op, name);
  CHECK(c.page_size >= 1, SA_ERR_SHAPE, "%s: %s.page_size must be >= 1", op, name);
  CHECK(c.max_pages >= 1, SA_ERR_SHAPE, "%s: %s.max_pages must be >= 1", op, name);
  CHECK(c.row_stride >= min_row_bytes, SA_ERR_SHAPE,
        "%s: %s.row_stride (%lld) < bytes of one row (%lld)", op, name, (long long)c.row_stride,
        (long long)min_row_bytes);
  CHECK(c.row_stride % 16 == 0 && aligned16(c.data), SA_ERR_SHAPE,
        "%s: %s.data and row_stride must be 16-byte aligned", op, name);
  CHECK(c.row_stride < (int64_t(1) << 31) && c.scale_stride >= 0 &&
            c.scale_stride < (int64_t(1) << 31),
        SA_ERR_SHAPE, "%s: %s.row_stride and scale_stride must be below 2^31", op, name);
  return SA_OK;
}

sa::CacheDev to_dev(const sa_cache& c) {
  sa::CacheDev d;
  d.data = reinterpret_cast<const char*>(c.data);
  d.scale = c.scale;
  d.block_table = c.block_table;
  d.row_stride = c.row_stride;
  d.scale_stride = c.scale_stride;
  d.page_size = c.page_size;
  d.page_shift = -1;
  if ((c.page_size & (c.page_size - 1)) == 0) {
    int s = 0;
    while ((1 << s) < c.page_size) ++s;
    d.page_shift = s;
  }
  d.max_pages = c.max_pages;
  d.pad = 0;
  return d;
}

sa_status hip_status(hipError_t e, const char* op) {
  if (e == hipSuccess) return SA_OK;
  return fail(SA_ERR_HIP, "%s: HIP error %d (%s)", op, (int)e, hipGetErrorString(e));
}

// ------------------------------------------------------------ index score
sa_status validate_index(const sa_index_desc* d, sa::IndexArgs* out) {
  const char* op = "sparse_index_score";
  CHECK(d, SA_ERR_NULL, "%s: desc is NULL", op);
  sa_status st = check_rows(d->rows, op);
  if (st) return st;
  CHECK(d->n_heads >= 1 && d->dim >= 1, SA_ERR_SHAPE, "%s: n_heads and dim must be >= 1", op);
  const int eb = elem_bytes(d->k.dtype);
  CHECK(eb > 0, SA_ERR_DTYPE, "%s: k.dtype must be F32, BF16 or FP8_E4M3", op);
  if (d->k.dtype == SA_F32) {
    CHECK(d->n_heads * d->dim + d->n_heads <= 12288, SA_ERR_UNSUPPORTED,
          "%s: F32 needs n_heads*dim <= 12288", op);
  } else {
    CHECK(d->dim == 64 || d->dim == 128, SA_ERR_UNSUPPORTED, "%s: BF16/FP8 need dim 64 or 128",
          op);
    CHECK(d->n_heads <= 64, SA_ERR_UNSUPPORTED, "%s: at most 64 index heads", op);
  }
  CHECK(d->k.heads == 1 && d->k.width == d->dim, SA_ERR_SHAPE,
        "%s: k must have heads == 1 and width == dim", op);
  CHECK(d->row_block >= 0, SA_ERR_SHAPE, "%s: row_block must be >= 0", op);
  CHECK(d->reserved == 0, SA_ERR_SHAPE, "%s: reserved must be 0", op);
  if (d->rows.n_rows == 0) return SA_OK;
  CHECK(d->q && d->w && (d->scores || d->sel), SA_ERR_NULL,
        "%s: q, w and scores (or sel) are required", op);
  CHECK(aligned16(d->q), SA_ERR_SHAPE, "%s: q must be 16-byte aligned", op);
  st = check_cache(d->k, op, "k", (int64_t)d->dim * eb);
  if (st) return st;
  CHECK(d->skip_k >= 0, SA_ERR_SHAPE, "%s: skip_k must be >= 0", op);
  if (d->cand) {
    CHECK(d->cand_count, SA_ERR_NULL, "%s: cand_count is required with cand", op);
    CHECK(d->cand_stride >= 1 && d->score_stride >= d->cand_stride, SA_ERR_SHAPE,
          "%s: need 1 <= cand_stride <= score_stride", op);
    CHECK(d->skip_k == 0, SA_ERR_SHAPE, "%s: skip_k (the dense route) needs full mode", op);
  } else {
    CHECK(d->score_stride >= 1, SA_ERR_SHAPE, "%s: score_stride must be >= 1", op);
  }
  if (out) {
    out->rows = to_dev(d->rows);
    out->k = to_dev(d->k);
    out->q = d->q;
    out->w = d->w;
    out->cand = d->cand;
    out->cand_count = d->cand_count;
    out->scores = d->scores;
    out->score_stride = d->score_stride;
    out->cand_stride = d->cand_stride;
    out->n_heads = d->n_heads;
    out->dim = d->dim;
    out->dtype = d->k.dtype;
    out->n_slots = d->cand ? d->cand_stride : (int32_t)d->score_stride;
    out->skip_k = d->skip_k;
  }
  return SA_OK;
}

// ----------------------------------------------------------------- select
sa_status validate_topk(const sa_topk_desc* d, sa::SelectArgs* out) {
  const char* op = "sparse_topk_select";
  CHECK(d, SA_ERR_NULL, "%s: desc is NULL", op);
  sa_status st = check_rows(d->rows, op);
  if (st) return st;
  CHECK(d->k >= 0, SA_ERR_SHAPE, "%s: k must be >= 0", op);
  const bool pool = d->pool != nullptr;
  CHECK(d->k > 0 || pool, SA_ERR_SHAPE, "%s: nothing to do (k == 0 and no pool)", op);
  if (d->rows.n_rows == 0) return SA_OK;
  CHECK(d->scores, SA_ERR_NULL, "%s: scores is required", op);
  CHECK(d->score_stride >= 1, SA_ERR_SHAPE, "%s: score_stride must be >= 1", op);
  if (d->k > 0) {
    CHECK(d->idx && d->count, SA_ERR_NULL, "%s: idx and count are required when k > 0", op);
    CHECK(d->idx_stride >= d->k, SA_ERR_SHAPE, "%s: idx_stride < k", op);
  }
  if (d->cand) {
    CHECK(d->cand_count, SA_ERR_NULL, "%s: cand_count is required with cand", op);
    CHECK(d->cand_stride >= 1 && d->cand_stride <= d->score_stride, SA_ERR_SHAPE,
          "%s: need 1 <= cand_stride <= score_stride", op);
    CHECK(!pool, SA_ERR_UNSUPPORTED, "%s: the block pool needs full-domain scores", op);
  }
  CHECK(d->score_stride <= (1 << 21), SA_ERR_UNSUPPORTED,
        "%s: at most 2097152 elements per row", op);
  if (pool) {
    CHECK(d->pool_count, SA_ERR_NULL, "%s: pool_count is required with pool", op);
    CHECK(d->block >= 1 && d->max_blocks >= 1, SA_ERR_SHAPE,
          "%s: block and max_blocks must be >= 1", op);
    CHECK((int64_t)d->pool_stride >= (int64_t)d->max_blocks * d->block, SA_ERR_SHAPE,
          "%s: pool_stride < max_blocks * block", op);
    CHECK(d->max_blocks <= 2048, SA_ERR_UNSUPPORTED, "%s: at most 2048 pool blocks", op);
  }
  if (out) {
    out->rows = to_dev(d->rows);
    out->scores = d->scores;
    out->score_stride = d->score_stride;
    out->cand = d->cand;
    out->cand_count = d->cand_count;
    out->cand_stride = d->cand_stride;
    out->k = d->k;
    out->idx = d->idx;
    out->count = d->count;
    out->idx_stride = d->idx_stride;
    out->block = pool ? d->block : 0;
    out->max_blocks = d->max_blocks;
    out->pool_stride = d->pool_stride;
    out->pool = d->pool;
    out->pool_count = d->pool_count;
    out->max_elems = d->cand ? d->cand_stride : (int32_t)d->score_stride;
    out->beta = nullptr;
    out->beta_stride = pool ? ((d->score_stride + d->block - 1) / d->block + 63) / 64 * 64 : 0;
  }
  return SA_OK;
}

// ------------------------------------------------------- fused selection
// sparse_index_score with sel: the rows per pass, the selection's arguments
// for a pass of that many rows, and the workspace (one pass's scores, then
// the selection's own workspace).
size_t align256(size_t b) { return (b + 255) / 256 * 256; }

struct FusedPlan {
  int rb;              // rows per pass
  sa::SelectArgs sel;  // for a pass of rb rows (pointers of the first pass)
  size_t score_bytes;  // one pass's scores, rounded up to 256 bytes
  size_t sel_bytes;    // the selection's workspace for rb rows
};

sa_status validate_fused(const sa_index_desc* d, FusedPlan* plan) {
  const char* op = "sparse_index_score";
  CHECK(d->sel, SA_ERR_NULL, "%s: sel is NULL", op);
  const int R = d->rows.n_rows;
  const int rb = (d->row_block > 0 && d->row_block < R) ? d->row_block : R;
  sa_topk_desc t = *d->sel;
  t.rows = d->rows;
  t.rows.n_rows = rb;
  // stands in for the pass's score buffer (replaced at launch)
  t.scores = reinterpret_cast<const float*>(uintptr_t(256));
  t.score_stride = d->score_stride;
  t.cand = d->cand;
  t.cand_count = d->cand_count;
  t.cand_stride = d->cand_stride;
  sa_status st = validate_topk(&t, &plan->sel);
  if (st) return st;
  plan->rb = rb;
  plan->score_bytes = align256((size_t)rb * (size_t)d->score_stride * sizeof(float));
  plan->sel_bytes = rb > 0 ? sa::topk_workspace_bytes(plan->sel) : 0;
  return SA_OK;
}

// -------------------------------------------------------------- attention
sa_status validate_attn(const sa_attn_desc* d, sa::AttnArgs* out) {
  const char* op = "sparse_attn_gather_fwd";
  CHECK(d, SA_ERR_NULL, "%s: desc is NULL", op);
  sa_status st = check_rows(d->rows, op);
  if (st) return st;
  CHECK(d->n_qsets >= 1, SA_ERR_SHAPE, "%s: n_qsets must be >= 1", op);
  const int hkv = d->k.heads, dqk = d->k.width, dv = d->d_v;
  CHECK(hkv >= 1 && d->n_heads_q >= hkv && d->n_heads_q % hkv == 0, SA_ERR_SHAPE,
        "%s: n_heads_q must be a positive multiple of k.heads", op);
  CHECK(dqk >= 1 && dv >= 1, SA_ERR_SHAPE, "%s: k.width and d_v must be >= 1", op);
  int kv_kind;
  if (d->k.dtype == SA_FP4_E2M1) {
    CHECK(d->v_from_k, SA_ERR_UNSUPPORTED, "%s: FP4 K needs v_from_k", op);
    kv_kind = 2;
  } else {
    kv_kind = d->v_from_k ? 1 : 0;
  }
  if (d->v_from_k) CHECK(dv <= dqk, SA_ERR_SHAPE, "%s: v_from_k needs d_v <= k.width", op);
  const int cdt = d->k.dtype == SA_FP4_E2M1 ? SA_BF16 : d->k.dtype;
  CHECK(cdt == SA_F32 || cdt == SA_BF16, SA_ERR_DTYPE, "%s: K must be F32, BF16 or FP4_E2M1", op);
  CHECK(d->q_dtype == cdt, SA_ERR_DTYPE, "%s: q_dtype must match the K compute type", op);
  CHECK(d->o_dtype == SA_F32 || d->o_dtype == SA_BF16, SA_ERR_DTYPE, "%s: o_dtype must be F32 or BF16",
        op);
  if (cdt == SA_F32) {
    CHECK(dqk <= 1024 && dv <= 256, SA_ERR_UNSUPPORTED, "%s: F32 needs k.width <= 1024, d_v <= 256",
          op);
  } else {
    const bool ok = (kv_kind == 0 && ((dqk == 128 && dv == 128) || (dqk == 256 && dv == 256))) ||
                    (kv_kind == 1 && ((dqk == 576 && dv == 512) || (dqk == 512 && dv == 512) ||
                                      (dqk == 128 && dv == 128))) ||
                    (kv_kind == 2 && dqk == 512 && dv == 512);
    CHECK(ok, SA_ERR_UNSUPPORTED, "%s: no kernel for k.width=%d d_v=%d (kv kind %d)", op, dqk, dv,
          kv_kind);
  }
  if (d->rows.n_rows == 0) return SA_OK;
  CHECK(d->q && d->o, SA_ERR_NULL, "%s: q and o are required", op);
  CHECK(aligned16(d->q) && aligned16(d->o), SA_ERR_SHAPE, "%s: q and o must be 16-byte aligned", op);
  if (kv_kind == 2) {
    st = check_cache(d->k, op, "k", (int64_t)hkv * dqk / 2);
    if (st) return st;
    CHECK(d->k.scale, SA_ERR_NULL, "%s: FP4 k needs k.scale", op);
    CHECK(d->k.scale_stride >= (int64_t)hkv * dqk / 16, SA_ERR_SHAPE, "%s: k.scale_stride too small",
          op);
    CHECK(d->k.scale_stride % 2 == 0 && ((uintptr_t)d->k.scale & 1u) == 0, SA_ERR_SHAPE,
          "%s: k.scale and k.scale_stride must be 2-byte aligned", op);
  } else {
    st = check_cache(d->k, op, "k", (int64_t)hkv * dqk * elem_bytes(cdt));
    if (st) return st;
  }
  if (kv_kind == 0) {
    st = check_cache(d->v, op, "v", (int64_t)hkv * dv * elem_bytes(cdt));
    if (st) return st;
    CHECK(d->v.dtype == d->k.dtype && d->v.heads == hkv && d->v.width == dv, SA_ERR_SHAPE,
          "%s: v must match k in dtype and heads, with width d_v", op);
    CHECK(d->v.block_table == d->k.block_table && d->v.page_size == d->k.page_size &&
              d->v.max_pages == d->k.max_pages,
          SA_ERR_SHAPE, "%s: k and v must share one page table", op);
  }
  if (d->idx) {
    CHECK(d->count, SA_ERR_NULL, "%s: count is required with idx", op);
    CHECK(d->idx_stride >= 1, SA_ERR_SHAPE, "%s: idx_stride must be >= 1", op);
  }
  CHECK((int64_t)d->rows.window + (d->idx ? d->idx_stride : 0) <= 131072, SA_ERR_UNSUPPORTED,
        "%s: window + idx_stride above 131072 entries per row", op);
  CHECK(!d->gate || aligned16(d->gate), SA_ERR_SHAPE, "%s: gate must be 16-byte aligned", op);
  CHECK(!d->gate || dv % 8 == 0, SA_ERR_UNSUPPORTED, "%s: a gate needs d_v divisible by 8", op);
  if (out) {
    out->rows = to_dev(d->rows);
    out->k = to_dev(d->k);
    out->v = to_dev(kv_kind == 0 ? d->v : d->k);
    out->q = d->q;
    out->idx = d->idx;
    out->count = d->count;
    out->o = d->o;
    out->lse = d->lse;
    out->part = nullptr;
    out->sink = d->sink;
    out->gate = d->gate;
    out->scale_log2 = d->scale * sa::kLog2e;
    out->idx_stride = d->idx ? d->idx_stride : 0;
    out->n_qsets = d->n_qsets;
    out->hq = d->n_heads_q;
    out->hkv = hkv;
    out->dqk = dqk;
    out->dv = dv;
    out->kv_kind = kv_kind;
    out->dtype = cdt;
    out->o_dtype = d->o_dtype;
    out->max_entries = d->rows.window + (d->idx ? d->idx_stride : 0);
    sa::attn_plan(*out);
  }
  return SA_OK;
}

}  // namespace

extern "C" {

sa_status sparse_index_score(const sa_index_desc* desc, void* ws, size_t ws_bytes, void* stream) {
  const char* op = "sparse_index_score";
  sa::IndexArgs a;
  sa_status st = validate_index(desc, &a);
  if (st || desc->rows.n_rows == 0) return st;
  const hipStream_t s = (hipStream_t)stream;
  if (!desc->sel) return hip_status(sa::launch_index_score(a, s), op);

  // Fused selection: score a pass of rows into the workspace, select on it.
  FusedPlan plan;
  st = validate_fused(desc, &plan);
  if (st) return st;
  const size_t need = plan.score_bytes + plan.sel_bytes;
  CHECK(ws && ws_bytes >= need, SA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given",
        op, need, ws_bytes);
  CHECK(((uintptr_t)ws & 255u) == 0, SA_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned",
        op);
  float* pass_scores = reinterpret_cast<float*>(ws);
  const int R = desc->rows.n_rows, rb = plan.rb;
  const size_t q_row = (size_t)desc->n_heads * desc->dim * elem_bytes(desc->k.dtype);
  for (int lo = 0; lo < R; lo += rb) {
    const int n = R - lo < rb ? R - lo : rb;
    sa::IndexArgs ia = a;
    ia.rows.n_rows = n;
    ia.rows.seq_of_row = a.rows.seq_of_row + lo;
    ia.rows.pos_of_row = a.rows.pos_of_row + lo;
    ia.q = reinterpret_cast<const char*>(a.q) + (size_t)lo * q_row;
    ia.w = a.w + (size_t)lo * desc->n_heads;
    if (a.cand) {
      ia.cand = a.cand + (size_t)lo * a.cand_stride;
      ia.cand_count = a.cand_count + lo;
    }
    ia.scores = pass_scores;
    st = hip_status(sa::launch_index_score(ia, s), op);
    if (st) return st;
    sa::SelectArgs sl = plan.sel;
    sl.rows = ia.rows;
    sl.scores = pass_scores;
    sl.cand = ia.cand;
    sl.cand_count = ia.cand_count;
    if (sl.k > 0) {
      sl.idx = plan.sel.idx + (size_t)lo * sl.idx_stride;
      sl.count = plan.sel.count + lo;
    }
    if (sl.pool) {
      sl.pool = plan.sel.pool + (size_t)lo * sl.pool_stride;
      sl.pool_count = plan.sel.pool_count + lo;
    }
    sl.beta = plan.sel_bytes ? reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + plan.score_bytes)
                             : nullptr;
    st = hip_status(sa::launch_topk_select(sl, s), op);
    if (st) return st;
  }
  return SA_OK;
}

sa_status sparse_topk_select(const sa_topk_desc* desc, void* ws, size_t ws_bytes, void* stream) {
  sa::SelectArgs a;
  sa_status st = validate_topk(desc, &a);
  if (st || desc->rows.n_rows == 0) return st;
  const size_t need = sa::topk_workspace_bytes(a);
  if (need) {
    CHECK(ws && ws_bytes >= need, SA_ERR_WORKSPACE,
          "sparse_topk_select: workspace of %zu bytes needed, %zu given", need, ws_bytes);
    CHECK(((uintptr_t)ws & 255u) == 0, SA_ERR_WORKSPACE,
          "sparse_topk_select: workspace must be 256-byte aligned");
    a.beta = reinterpret_cast<float*>(ws);
  }
  return hip_status(sa::launch_topk_select(a, (hipStream_t)stream), "sparse_topk_select");
}

sa_status sparse_attn_gather_fwd(const sa_attn_desc* desc, void* ws, size_t ws_bytes,
                                 void* stream) {
  sa::AttnArgs a;
  sa_status st = validate_attn(desc, &a);
  if (st || desc->rows.n_rows == 0) return st;
  const size_t need = sa::attn_workspace_bytes(a);
  if (need) {
    CHECK(ws && ws_bytes >= need, SA_ERR_WORKSPACE,
          "sparse_attn_gather_fwd: workspace of %zu bytes needed, %zu given", need, ws_bytes);
    CHECK(((uintptr_t)ws & 255u) == 0, SA_ERR_WORKSPACE,
          "sparse_attn_gather_fwd: workspace must be 256-byte aligned");
    a.part = reinterpret_cast<float*>(ws);
  }
  return hip_status(sa::launch_attn_gather(a, (hipStream_t)stream), "sparse_attn_gather_fwd");
}

sa_status sparse_attn_score(const sa_attn_desc* d, float* scores, int64_t score_stride,
                            void* stream) {
  const char* op = "sparse_attn_score";
  CHECK(d, SA_ERR_NULL, "%s: desc is NULL", op);
  sa_status st = check_rows(d->rows, op);
  if (st) return st;
  CHECK(d->n_qsets >= 1, SA_ERR_SHAPE, "%s: n_qsets must be >= 1", op);
  const int hkv = d->k.heads, dqk = d->k.width;
  CHECK(hkv >= 1 && d->n_heads_q >= hkv && d->n_heads_q % hkv == 0, SA_ERR_SHAPE,
        "%s: n_heads_q must be a positive multiple of k.heads", op);
  CHECK(d->k.dtype == SA_F32 || d->k.dtype == SA_BF16, SA_ERR_DTYPE, "%s: K must be F32 or BF16",
        op);
  CHECK(d->q_dtype == d->k.dtype, SA_ERR_DTYPE, "%s: q_dtype must match k.dtype", op);
  if (d->k.dtype == SA_BF16) {
    CHECK(dqk == 64 || dqk == 128, SA_ERR_UNSUPPORTED, "%s: BF16 needs k.width 64 or 128", op);
    CHECK(8 % hkv == 0, SA_ERR_UNSUPPORTED, "%s: BF16 needs k.heads dividing 8", op);
    CHECK(d->n_qsets * (d->n_heads_q / hkv) <= 16, SA_ERR_UNSUPPORTED,
          "%s: BF16 needs n_qsets * (n_heads_q / k.heads) <= 16", op);
  } else {
    CHECK((int64_t)d->n_qsets * d->n_heads_q * (dqk + 1) <= 16384, SA_ERR_UNSUPPORTED,
          "%s: F32 needs n_qsets * n_heads_q * (k.width + 1) <= 16384", op);
  }
  if (d->rows.n_rows == 0) return SA_OK;
  CHECK(d->q && d->lse && scores, SA_ERR_NULL, "%s: q, lse and scores are required", op);
  CHECK(aligned16(d->q), SA_ERR_SHAPE, "%s: q must be 16-byte aligned", op);
  CHECK(score_stride >= 1, SA_ERR_SHAPE, "%s: score_stride must be >= 1", op);
  st = check_cache(d->k, op, "k", (int64_t)hkv * dqk * elem_bytes(d->k.dtype));
  if (st) return st;
  sa::ScoreArgs a;
  a.rows = to_dev(d->rows);
  a.k = to_dev(d->k);
  a.q = d->q;
  a.lse = d->lse;
  a.scores = scores;
  a.score_stride = score_stride;
  a.scale_log2 = d->scale * sa::kLog2e;
  a.n_qsets = d->n_qsets;
  a.hq = d->n_heads_q;
  a.hkv = hkv;
  a.dqk = dqk;
  a.dtype = d->k.dtype;
  a.n_slots = (int32_t)score_stride;
  return hip_status(sa::launch_attn_score(a, (hipStream_t)stream), op);
}

sa_status sparse_check_indices(const sa_topk_desc* desc, uint32_t* err, void* stream) {
  const char* op = "sparse_check_indices";
  CHECK(desc, SA_ERR_NULL, "%s: desc is NULL", op);
  CHECK(err, SA_ERR_NULL, "%s: err is NULL", op);
  sa_status st = check_rows(desc->rows, op);
  if (st) return st;
  CHECK(desc->k >= 1, SA_ERR_SHAPE, "%s: k must be >= 1", op);
  if (desc->rows.n_rows > 0) {
    CHECK(desc->idx && desc->count, SA_ERR_NULL, "%s: idx and count are required", op);
    CHECK(desc->idx_stride >= desc->k, SA_ERR_SHAPE, "%s: idx_stride < k", op);
  }
  sa::CheckArgs a;
  a.rows = to_dev(desc->rows);
  a.idx = desc->idx;
  a.count = desc->count;
  a.err = err;
  a.idx_stride = desc->idx_stride;
  a.k = desc->k;
  a.candidate_mode = desc->cand != nullptr;
  return hip_status(sa::launch_check_indices(a, (hipStream_t)stream), op);
}

sa_status sparse_attn_gather_fwd_noalloc(const sa_attn_desc* desc, void* stream) {
  const char* op = "sparse_attn_gather_fwd_noalloc";
  sa::AttnArgs a;
  sa_status st = validate_attn(desc, &a);
  if (st || desc->rows.n_rows == 0) return st;
  const size_t need = sa::attn_workspace_bytes(a);
  CHECK(need <= sa::kNoAllocScratchBytes, SA_ERR_WORKSPACE,
        "%s: the call needs %zu bytes of split partials, above the %zu-byte static scratch", op,
        need, sa::kNoAllocScratchBytes);
  return hip_status(sa::launch_attn_gather_noalloc(a, (hipStream_t)stream), op);
}

size_t sa_workspace_size(int32_t op, const void* desc) {
  switch (op) {
    case SA_OP_INDEX_SCORE: {
      const sa_index_desc* d = reinterpret_cast<const sa_index_desc*>(desc);
      if (validate_index(d, nullptr)) return (size_t)-1;
      if (!d->sel || d->rows.n_rows == 0) return 0;
      FusedPlan plan;
      if (validate_fused(d, &plan)) return (size_t)-1;
      return plan.score_bytes + plan.sel_bytes;
    }
    case SA_OP_TOPK_SELECT: {
      const sa_topk_desc* d = reinterpret_cast<const sa_topk_desc*>(desc);
      sa::SelectArgs a;
      if (validate_topk(d, &a)) return (size_t)-1;
      if (d->rows.n_rows == 0) return 0;
      return sa::topk_workspace_bytes(a);
    }
    case SA_OP_ATTN_GATHER_FWD: {
      const sa_attn_desc* d = reinterpret_cast<const sa_attn_desc*>(desc);
      sa::AttnArgs a;
      if (validate_attn(d, &a)) return (size_t)-1;
      if (d->rows.n_rows == 0) return 0;
      return sa::attn_workspace_bytes(a);
    }
    default:
      fail(SA_ERR_SHAPE, "sa_workspace_size: unknown op %d", op);
      return (size_t)-1;
  }
}

const char* sa_last_error(void) { return g_err; }

int32_t sa_abi_version(void) { return (SA_ABI_VERSION << 16) | SA_INDEX_FORMAT; }

}  // extern "C"
