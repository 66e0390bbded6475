// Internal launch interface between the C ABI layer (abi.cpp) and the gfx950
// kernels.  Host-side only; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace sa {

// ----------------------------------------------------------------- indexer
struct IndexArgs {
  RowsDev rows;
  CacheDev k;
  const void* q;        // [R][n_heads][dim]
  const float* w;       // [R][n_heads]
  const int32_t* cand;  // optional [R][cand_stride]
  const int32_t* cand_count;
  float* scores;
  int64_t score_stride;
  int32_t cand_stride;
  int32_t n_heads;
  int32_t dim;
  int32_t dtype;        // SA_F32 / SA_BF16 / SA_FP8_E4M3
  int32_t n_slots;      // score slots per row to cover (grid extent)
  int32_t skip_k;       // dense route: rows with n_avail - window <= skip_k get 0s
};
hipError_t launch_index_score(const IndexArgs& a, hipStream_t s);

// ------------------------------------------------------------------ select
struct SelectArgs {
  RowsDev rows;
  const float* scores;
  int64_t score_stride;
  const int32_t* cand;
  const int32_t* cand_count;
  int32_t cand_stride;
  int32_t k;
  int32_t* idx;
  int32_t* count;
  int32_t idx_stride;
  int32_t block;
  int32_t max_blocks;
  int32_t pool_stride;
  int32_t* pool;
  int32_t* pool_count;
  int32_t max_elems;  // upper bound on elements per row (picks the block size)
  float* beta;        // pool mode: block maxima [R][beta_stride] (workspace)
  int64_t beta_stride;
};
size_t topk_workspace_bytes(const SelectArgs& a);
hipError_t launch_topk_select(const SelectArgs& a, hipStream_t s);

// --------------------------------------------------------------- attention
struct AttnArgs {
  RowsDev rows;
  CacheDev k;
  CacheDev v;
  const void* q;        // [n_qsets][R][hq][dqk]
  const int32_t* idx;   // [R][idx_stride] or NULL
  const int32_t* count;
  void* o;              // [n_qsets][R][hq][dv]
  float* lse;           // [n_qsets][R][hq] or NULL
  float* part;          // split partials (workspace) or NULL
  const float* sink;    // [n_qsets][hq] sink logits (natural units) or NULL
  const void* gate;     // [n_qsets][R][hq][dv] output gate logits (dtype) or NULL
  float scale_log2;     // softmax scale * log2(e)
  int32_t idx_stride;
  int32_t n_qsets;
  int32_t hq;
  int32_t hkv;
  int32_t dqk;
  int32_t dv;
  int32_t kv_kind;      // 0 separate K/V, 1 V = first dv of K, 2 FP4 shared row
  int32_t dtype;        // SA_F32 or SA_BF16 (q, K, V, o compute type)
  int32_t o_dtype;
  int32_t n_split;      // entry-range splits (>= 1)
  int32_t max_entries;  // upper bound on window + selected entries per row
};
size_t attn_workspace_bytes(const AttnArgs& a);
void attn_plan(AttnArgs& a);  // fills n_split
hipError_t launch_attn_gather(const AttnArgs& a, hipStream_t s);
// The allocation-free variant: split partials in a static per-device array
// of kNoAllocScratchBytes (hipErrorInvalidValue if a call needs more).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t launch_attn_gather_noalloc(AttnArgs a, hipStream_t s);

// ------------------------------------------------- full-attention score
struct ScoreArgs {
  RowsDev rows;
  CacheDev k;
  const void* q;        // [n_qsets][R][hq][dqk]
  const float* lse;     // [n_qsets][R][hq] (natural log)
  float* scores;        // [R][score_stride]
  int64_t score_stride;
  float scale_log2;     // softmax scale * log2(e)
  int32_t n_qsets;
  int32_t hq;
  int32_t hkv;
  int32_t dqk;
  int32_t dtype;        // SA_F32 or SA_BF16
  int32_t n_slots;      // score slots per row to cover (grid extent)
};
hipError_t launch_attn_score(const ScoreArgs& a, hipStream_t s);

// ------------------------------------------------------------ index check
enum : uint32_t { kCheckCount = 1, kCheckDomain = 2, kCheckOrder = 3, kCheckPadding = 4 };
struct CheckArgs {
  RowsDev rows;
  const int32_t* idx;   // [R][idx_stride]
  const int32_t* count; // [R]
  uint32_t* err;        // one word: (row << 3) | code of the first failure, or ~0
  int32_t idx_stride;
  int32_t k;
  int32_t candidate_mode;  // 1: entries anywhere in [0, n_avail) outside the window
};
hipError_t launch_check_indices(const CheckArgs& a, hipStream_t s);

}  // namespace sa
