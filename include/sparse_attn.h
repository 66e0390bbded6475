/*
 * sparse_attn.h -- C ABI of the MI355X (gfx950) library for indexer-driven
 * top-k sparse attention with index reuse.
 *
 * The path has three steps, one entry point each:
 *
 *   sparse_index_score     the lightning-indexer score of every visible cache
 *                          entry (or of a candidate list) for each query row
 *                          ["Lecture 10 - Hybrid LLMs", section 5.1, the indexer
 *                          equation; "CSA, HCA and CSA2", section 3.2,
 *                          Reindex scores only the candidate pool];
 *   sparse_topk_select     the top-k entries outside a forced recent window,
 *                          and/or the block-max candidate pool
 *                          ["HySparse2", section 7.2; "CSA, HCA and CSA2",
 *                          section 3.2, Hierarchical Sparse Indexer];
 *   sparse_attn_gather_fwd one joint softmax over window + selected entries,
 *                          gathered by index from one shared paged KV cache,
 *                          for several query sets at once
 *                          ["HySparse2", sections 5 and 7.2: the SA layers reuse
 *                          the FA layer's KV and indices with their own
 *                          queries; "CSA, HCA and CSA2", section 3.1: Reuse
 *                          layers read the existing indices].
 *
 * Index reuse needs no entry point: an index tensor written by
 * sparse_topk_select is passed unchanged to any number of
 * sparse_attn_gather_fwd calls.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer inside a descriptor is DEVICE memory owned by the caller,
 *    unless stated otherwise.  The library never allocates, frees or keeps a
 *    pointer after the call returns.  Scratch memory comes only from the
 *    caller's workspace `ws` of `ws_bytes` bytes (device memory, 256-byte
 *    aligned), whose required size sa_workspace_size() reports.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  Buffers must stay alive until the stream work completes.
 *  - Descriptors are read on the host during the call only.
 *  - No exception crosses the ABI.  Host-side validation failures return a
 *    negative sa_status and leave outputs untouched; sa_last_error() gives a
 *    thread-local message.  Index CONTENTS are trusted: -1 means padding, any
 *    other value must be a visible entry of the row (sparse_check_indices
 *    verifies a tensor on the device when a caller wants it checked).
 *  - The library keeps no state between calls and is reentrant; concurrent
 *    calls must use distinct workspaces.
 *
 * Rows, domain and window
 * -----------------------
 * Query row r belongs to sequence b = seq_of_row[r] at token position
 * t = pos_of_row[r].  A cache entry covers `stride` consecutive tokens
 * (stride 1 = one entry per token); entry e is visible to the row iff every
 * token it covers is visible: stride*(e+1) <= min(t+1, seq_len[b]).  The
 * visible entries are therefore e < n_avail = floor(min(t+1, seq_len[b]) /
 * stride) ("CSA, HCA and CSA2", section 2.2: no query reads an entry holding a
 * future token; a partial tail entry is masked).  The window is the last
 * `window` visible entries, W = [max(0, n_avail - window), n_avail); the
 * candidates for top-k selection are the visible entries before it.  A row
 * with b < 0 or t < 0 is padding and sees nothing.
 *
 * Paged caches
 * ------------
 * Entry e of sequence b lives in page p = block_table[b * max_pages +
 * e / page_size] (or p = b * max_pages + e / page_size when block_table is
 * NULL) at slot u = p * page_size + e % page_size (u must be below 2^31);
 * its bytes start at data + u * row_stride.  Every visible entry must be backed by the cache
 * (n_avail <= max_pages * page_size); the kernels do not check this.  Within a row, head h channel c is element
 * h * width + c ("Lecture 10", section 5.5: a sparse kernel fetches entries by
 * index, through the block table when paged; "HySparse2", section 7.2: no
 * concatenated copy is made).
 *
 * Index format (part of the compatibility contract, "CSA, HCA and CSA2",
 * prefix-cache keying discussion): int32 entry indices, ascending, -1 padded,
 * with a per-row count; ties in score go to the LOWER index; -0 equals +0.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_ABI_VERSION 3       /* bumped on any descriptor layout change   */
#define SA_INDEX_FORMAT 1      /* int32 asc, -1 pad, lowest-index tie-break */

typedef int32_t sa_status;
enum {
  SA_OK = 0,
  SA_ERR_NULL = -1,        /* a required pointer is NULL                    */
  SA_ERR_SHAPE = -2,       /* sizes, strides or alignment inconsistent       */
  SA_ERR_DTYPE = -3,       /* unsupported dtype or dtype combination        */
  SA_ERR_UNSUPPORTED = -4, /* valid request the library has no kernel for  */
  SA_ERR_WORKSPACE = -5,   /* ws too small or misaligned                    */
  SA_ERR_HIP = -6          /* a HIP runtime call or launch failed           */
};

typedef enum {
  SA_F32 = 0,      /* IEEE binary32                                          */
  SA_BF16 = 1,     /* bfloat16                                               */
  SA_FP8_E4M3 = 2, /* OCP FP8 E4M3 (e4m3fn)                                  */
  SA_FP4_E2M1 = 3  /* FP4 E2M1, two channels per byte (even channel in the low
                      nibble) with one E4M3 scale byte per 16 channels
                      ("CSA, HCA and CSA2", section 3.2)                     */
} sa_dtype;

/* A paged cache of rows (see "Paged caches" above). */
typedef struct {
  const void* data;          /* row pool                                      */
  const uint8_t* scale;      /* SA_FP4_E2M1 only: E4M3 scale pool, one byte per
                                16 channels, row u at scale + u*scale_stride;
                                NULL otherwise                                 */
  const int32_t* block_table;/* [n_seqs][max_pages] page ids, or NULL          */
  int32_t page_size;         /* entries per page (>= 1)                       */
  int32_t max_pages;         /* pages per sequence in block_table             */
  int32_t heads;             /* heads per row                                 */
  int32_t width;             /* channels per head                             */
  int64_t row_stride;        /* bytes between consecutive slots (16-B aligned,
                                below 2^31)                                    */
  int64_t scale_stride;      /* bytes between consecutive scale rows (below
                                2^31)                                          */
  int32_t dtype;             /* sa_dtype                                      */
  int32_t reserved;
} sa_cache;

/* The query rows of a call (see "Rows, domain and window" above). */
typedef struct {
  int32_t n_rows;            /* R                                             */
  int32_t n_seqs;            /* B                                             */
  const int32_t* seq_of_row; /* [R]                                           */
  const int32_t* pos_of_row; /* [R] token position t                          */
  const int32_t* seq_len;    /* [B] tokens in each sequence                   */
  int32_t stride;            /* tokens per cache entry (>= 1)                 */
  int32_t window;            /* forced recent window w (>= 0), in entries     */
} sa_rows;

/*
 * sparse_index_score -- lightning-indexer scores
 * ["Lecture 10 - Hybrid LLMs", section 5.1]:
 *
 *   score[r][s] = sum_{j < n_heads} w[r][j] * ReLU( q[r][j][:] . k[s][:] )
 *
 * for every visible entry s of row r (window included), or, when `cand` is
 * given, for s = cand[r][i], i < cand_count[r] (Reindex: "CSA, HCA and CSA2",
 * section 3.2 -- only the pool is rescored, with this layer's own q and w).
 *
 *   q        [R][n_heads][dim], dtype = k.dtype (F32, BF16 or FP8_E4M3)
 *   w        [R][n_heads] f32
 *   k        the index-key cache: heads = 1, width = dim, dtype as q
 *   scores   [R][score_stride] f32 out. Full mode writes scores[r][s] for
 *            s < n_avail(r); candidate mode writes scores[r][i] for
 *            i < cand_count[r] (-inf for a padding or invisible candidate).
 *            Other slots are not written.
 *   score_stride >= max n_avail (full) or >= cand_stride (candidate mode).
 *   skip_k   dense route (full mode only; 0 = off): a row with at most skip_k
 *            candidates (n_avail - window <= skip_k) is not scored -- a
 *            window + top-k selection with k >= skip_k keeps every candidate
 *            of such a row whatever its scores -- and gets scores[r][s] = 0
 *            for s < n_avail instead, without reading the cache ("Lecture
 *            10", section 5.5: when a row's context is no longer than the
 *            budget, sparse selection only adds the indexer's cost, so it
 *            falls back to dense attention; with k >= the candidates the
 *            selected set IS the dense set).
 *
 * Accumulation is fp32 (MFMA for BF16/FP8, FMA for F32); the ReLU and the
 * weighted head sum are fp32.
 *
 * Fused selection (sel != NULL): the scores feed the window + top-k selection
 * (and/or the block-max pool) directly, and the call writes the selection's
 * outputs instead of a score tensor ("CSA, HCA and CSA2", section 2.2: a
 * prefill must not hold the n x n_c score matrix; "Lecture 10", section 5.1:
 * the indexer's scores exist only to be ranked).  The rows are processed in
 * passes of row_block rows (0 = all rows in one pass): each pass scores its
 * rows into the workspace, then runs on them exactly the selection
 * sparse_topk_select would run with *sel.  So the outputs are identical to
 * the two calls made separately, and the workspace holds the scores of one
 * pass only (row_block * score_stride floats) plus the selection's own
 * workspace for row_block rows (sa_workspace_size(SA_OP_INDEX_SCORE, desc)).
 *   - From *sel the call reads k, idx, count, idx_stride, block, max_blocks,
 *     pool_stride, pool and pool_count (outputs for all R rows, as for
 *     sparse_topk_select); its rows, scores, score_stride, cand, cand_count
 *     and cand_stride are ignored: the rows and candidates are this
 *     descriptor's, and score_stride here gives the capacity of a pass's
 *     score rows (>= max n_avail, or >= cand_stride in candidate mode).
 *   - `scores` may be NULL and is not written.
 */
struct sa_topk_desc;

typedef struct {
  sa_rows rows;
  const void* q;
  const float* w;
  sa_cache k;
  int32_t n_heads;
  int32_t dim;
  const int32_t* cand;       /* optional [R][cand_stride], ascending, -1 pad  */
  const int32_t* cand_count; /* [R] when cand != NULL                         */
  int32_t cand_stride;
  int32_t skip_k;            /* dense route threshold (0 = off), see above     */
  float* scores;
  int64_t score_stride;
  const struct sa_topk_desc* sel;  /* optional fused selection, see above      */
  int32_t row_block;         /* fused selection: rows per pass (0 = all)      */
  int32_t reserved;          /* 0                                             */
} sa_index_desc;

/*
 * sparse_topk_select -- window + top-k, and the block-max pool.
 *
 * Token mode (k > 0) ["HySparse2", section 7.2]: the candidates are the
 * visible entries outside the window (candidate mode: the listed entries
 * outside the window).  The first min(k, #candidates) of them in the order
 * (score descending, index ascending; -0 == +0) are written ASCENDING to
 * idx[r][0 .. count[r]), and idx[r][count[r] .. k) = -1.
 *
 * Pool mode (pool != NULL, block >= 1, max_blocks <= 2048, full-domain scores
 * only) ["CSA, HCA and CSA2", section 3.2; "HySparse2", appendix A.1, the
 * first generation's 16 blocks of 64 tokens]: every aligned block j of
 * `block` entries gets beta_j = the max score over its candidates (visible
 * entries outside the window; with window 0, every visible member); the first
 * min(max_blocks, #blocks) blocks in the order (beta descending, j ascending)
 * are kept, and their candidates are written ascending to
 * pool[r][0 .. pool_count[r]), pool[r][pool_count[r] .. max_blocks*block) =
 * -1.  The pool is in the index format, so it can also serve directly as a
 * block-level selection (pool as idx, pool_count as count).
 *
 * Both modes can run in one call from the same scores.
 *
 *   scores      [R][score_stride] f32, as written by sparse_index_score
 *   cand/cand_count  candidate mode: scores[r][i] belongs to entry cand[r][i];
 *               the list must be ascending (the pool is)
 *   idx         [R][idx_stride] int32 out, idx_stride >= k;   count [R] out
 *   pool        [R][pool_stride] int32 out, pool_stride >= max_blocks*block;
 *               pool_count [R] out
 * Scores must not be NaN.
 *
 * Workspace: sa_workspace_size(SA_OP_TOPK_SELECT, desc) bytes.  Its contents
 * on entry are ignored (the call clears what it counts into), so one
 * workspace may serve any sequence of calls, of any entry point and any row
 * count, as long as no two of them overlap in time.
 */
typedef struct sa_topk_desc {
  sa_rows rows;
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
} sa_topk_desc;

/*
 * sparse_attn_gather_fwd -- one joint softmax over the window plus the
 * selected entries ["HySparse2", section 7.2], for n_qsets query sets that
 * share the KV cache and the index tensor ["HySparse2", section 5; "CSA, HCA
 * and CSA2", section 3.1].
 *
 * For query set i, row r, query head h with KV head g = h / (n_heads_q /
 * k.heads), over A = W(r) U {idx[r][0 .. count[r])}:
 *   logit_s = scale * q[i][r][h][:] . K[s][g][:]
 *   Z       = sum_s exp(logit_s) + exp(sink[i][h])      (no sink: 0 for that term)
 *   o[i][r][h][:] = sigmoid(gate[i][r][h][:]) * sum_s exp(logit_s) / Z * V[s][g][:]
 *   lse[i][r][h]  = log Z                              (natural log)
 * An empty A gives o = 0 and lse = sink (-inf without a sink).  Selected
 * entries must lie outside the window (sparse_topk_select guarantees it).
 *
 * The optional per-head sink bias and output sigmoid gate are those the
 * HySparse2 page lists around its core softmax ("HySparse2", section 17.1: every
 * SA layer has an output sigmoid gate and a learnable per-head sink bias).
 * The sink is a logit for a virtual entry whose value row is zero; the gate
 * multiplies each output channel.
 *   sink     optional [n_qsets][n_heads_q] f32 (each query set is a layer
 *            with its own parameters); NULL = no sink
 *   gate     optional [n_qsets][R][n_heads_q][d_v], dtype q_dtype; NULL = none
 *
 *   q        [n_qsets][R][n_heads_q][k.width], dtype q_dtype (F32 or BF16)
 *   k        key cache, heads = H_kv, width = d_qk; BF16, F32 or FP4_E2M1
 *   v        value cache, heads = H_kv, width = d_v, same dtype as k, and the
 *            SAME block_table pointer, page_size and max_pages as k (an
 *            entry's V row sits at the same slot as its K row); ignored when
 *            v_from_k != 0, in which case V is the first d_v
 *            channels of the K row (MLA latent / shared-row caches,
 *            "Lecture 10", section 5.1: one latent entry serves all heads)
 *   idx      [R][idx_stride] int32 (NULL: window only); count [R].
 *            window + idx_stride must not exceed 131072 entries
 *            (SA_ERR_UNSUPPORTED otherwise)
 *   o        [n_qsets][R][n_heads_q][d_v], dtype o_dtype (F32 or BF16)
 *   lse      optional [n_qsets][R][n_heads_q] f32
 * Softmax statistics and accumulation are fp32; BF16 / FP4 operands go
 * through MFMA (FP4 is dequantised exactly to bf16 in the kernel).
 */
typedef struct {
  sa_rows rows;
  int32_t n_qsets;
  int32_t n_heads_q;
  const void* q;
  int32_t q_dtype;
  int32_t d_v;
  sa_cache k;
  sa_cache v;
  int32_t v_from_k;
  int32_t idx_stride;
  const int32_t* idx;
  const int32_t* count;
  float scale;
  int32_t o_dtype;
  void* o;
  float* lse;
  const float* sink;         /* optional [n_qsets][n_heads_q], see above      */
  const void* gate;          /* optional [n_qsets][R][n_heads_q][d_v]          */
} sa_attn_desc;

enum { SA_OP_INDEX_SCORE = 0, SA_OP_TOPK_SELECT = 1, SA_OP_ATTN_GATHER_FWD = 2 };

/* Entry points.  `stream` is a hipStream_t. */
sa_status sparse_index_score(const sa_index_desc* desc, void* ws, size_t ws_bytes, void* stream);
sa_status sparse_topk_select(const sa_topk_desc* desc, void* ws, size_t ws_bytes, void* stream);
sa_status sparse_attn_gather_fwd(const sa_attn_desc* desc, void* ws, size_t ws_bytes,
                                 void* stream);

/*
 * sparse_attn_gather_fwd_noalloc -- sparse_attn_gather_fwd for callers that
 * cannot allocate or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same descriptor, same
 * kernels, same results; the split partials that sparse_attn_gather_fwd keeps
 * in `ws` live instead in one static device array of 64 MiB per GPU, which
 * the library holds until the process ends.  A call needing more partials
 * than that (sa_workspace_size(SA_OP_ATTN_GATHER_FWD, desc) > 64 MiB) returns
 * SA_ERR_WORKSPACE and launches nothing.  The call allocates and frees
 * nothing.  Every call on one GPU shares that GPU's array (nothing in it needs
 * to start at any value): calls that overlap in time on one GPU race.
 */
sa_status sparse_attn_gather_fwd_noalloc(const sa_attn_desc* desc, void* stream);

/*
 * sparse_attn_score -- the selection score of a full-attention layer
 * ["HySparse2", appendix A.1: the FA layer runs ordinary full attention and
 * picks the important history positions from its own attention scores, and
 * its SA layers reuse them; "Lecture 10", section 5.2: the per-position
 * target is the main attention summed over heads]:
 *
 *   scores[r][s] = sum_{i < n_qsets} sum_{h < n_heads_q}
 *                  exp( scale * q[i][r][h][:] . K[s][g][:] - lse[i][r][h] )
 *
 * for every visible entry s < n_avail(r) (g = h / (n_heads_q / k.heads)):
 * the probability each head gives s in dense attention over the row's
 * visible entries, summed over heads.  `lse` must be that dense attention's
 * log-normaliser, e.g. from sparse_attn_gather_fwd over the same rows with
 * rows.window >= every n_avail and idx = NULL.  The scores then feed
 * sparse_topk_select (window + top-k) like indexer scores do.
 *
 * Reads desc->rows (window ignored), n_qsets, n_heads_q, q, q_dtype, k, scale
 * and lse; the V, index and output fields are ignored.
 *   q       [n_qsets][R][n_heads_q][k.width], dtype = k.dtype (F32 or BF16)
 *   scores  [R][score_stride] f32 out; slots s >= n_avail(r) are not written.
 *           score_stride >= max n_avail.
 * BF16 needs k.width 64 or 128, k.heads dividing 8 and n_qsets * (n_heads_q /
 * k.heads) <= 16; F32 needs n_qsets * n_heads_q * (k.width + 1) <= 16384
 * (SA_ERR_UNSUPPORTED otherwise).  Logits and sums are fp32 (MFMA for BF16).
 */
sa_status sparse_attn_score(const sa_attn_desc* desc, float* scores, int64_t score_stride,
                            void* stream);

/*
 * sparse_check_indices -- device-side check of an index tensor before it is
 * reused ("CSA, HCA and CSA2", section 5.1, fault injection: a Reuse layer's
 * indices shifted by one token, or a leaked row, must be caught by an
 * assertion rather than by an output that merely looks plausible).
 *
 * Reads desc->rows, k, idx, idx_stride, count and cand (only whether it is
 * NULL); every other field is ignored.  Row r passes when 0 <= count[r] <= k,
 * idx[r][0 .. count) is strictly ascending and lies among the row's
 * candidates -- token mode (cand == NULL): [0, win_lo); candidate mode:
 * [0, n_avail) outside the window -- and idx[r][count .. k) == -1.  A padding
 * row passes only with count 0.
 *
 *   err  one device uint32 (caller-owned), written on `stream`: 0xFFFFFFFF if
 *        every row passes, else (r << 3) | code for the smallest failing row r
 *        and its smallest code: 1 count out of range, 2 index outside the
 *        candidates, 3 not strictly ascending, 4 padding slot not -1.
 *
 * Only idx, count and the row geometry are read, so any contents are safe to
 * check.  Returns SA_ERR_* for an invalid descriptor (err untouched).
 */
sa_status sparse_check_indices(const sa_topk_desc* desc, uint32_t* err, void* stream);

/* Workspace bytes `op` (SA_OP_*) needs for `desc` (a pointer to the matching
 * descriptor); 0 if none.  Returns (size_t)-1 if the descriptor is invalid. */
size_t sa_workspace_size(int32_t op, const void* desc);

/* Thread-local text for the last non-OK status returned on this thread. */
const char* sa_last_error(void);

/* (SA_ABI_VERSION << 16) | SA_INDEX_FORMAT */
int32_t sa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPARSE_ATTN_H */
