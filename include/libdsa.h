/*
 * libdsa -- the data-parallel hot path of DeepSeek Sparse Attention (DSA)
 * for AMD Instinct MI355X (gfx950).
 *
 * Three stages, each a HIP kernel family behind this C ABI:
 *   1. lightning-indexer scores   I[t,s] = scale * sum_j w[t,j] * ReLU(q[t,j] . k[s])
 *   2. per-query causal top-k     S_t = the min(k, n_t) best positions, ascending
 *   3. sparse MLA over S_t        absorbed (MQA) form with online softmax
 *
 * Sources (page title, section / equation):
 *   [G] "DeepSeek Sparse Attention DSA Architecture Guide":
 *       "Stage 1: The Lightning Indexer" -- the ReLU score equation and item 3
 *         (per-key separable scores; FP8 operands, item 1);
 *       "Stage 2: Fine-Grained Token Selection" -- the TopK, gather and u_t
 *         equations (softmax restricted to S_t);
 *       "The Classical Multi-Head Latent Attention (MLA) Mechanism" -- the
 *         latent + decoupled-rotary logit A_{t,s,i};
 *       "End-to-End Implementation" -- k = min(top_k, seq_len), selected
 *         positions re-sorted into ascending (temporal) order;
 *       the two-stage pipeline figure (indexer -> top-k -> selective fetch ->
 *         sparse MLA kernel).
 *   [P] "Sparse Attention in Large Language Models: Architecture Evolution
 *       and Engineering Practice", section 4.1 -- paged KV-cache storage.
 *
 * Conventions (the pages give none; these are the library's):
 *   - Every tensor pointer is a DEVICE pointer unless stated otherwise; the
 *     descriptor structs themselves are host memory, read during the call.
 *   - Layouts are row-major and densely packed as written ([a,b,c]: c fastest).
 *   - The caller owns all memory.  The library never allocates, frees or
 *     synchronises; every call only enqueues kernels on `stream` and returns.
 *   - Arguments are validated on the host before anything is launched; on a
 *     validation failure nothing is enqueued.  Shapes the kernels do not
 *     implement return DSA_ERR_UNSUPPORTED.  A failed launch returns
 *     DSA_ERR_HIP.  dsa_last_error() then describes the failure.
 *   - Device-side preconditions are documented, not checked: batch arrays
 *     consistent with the host-side bounds, indices in range, page ids
 *     valid, no NaN scores.
 *   - The library keeps no mutable global state, except the static scratch
 *     array of dsa_forward_noalloc: calls on different streams (or threads)
 *     may run concurrently if their buffers do not overlap (for
 *     dsa_forward_noalloc, see its note).
 *
 * Batch semantics.  Sequence b owns query rows q_seq_start[b] ..
 * q_seq_start[b+1]-1 and a key history of k_len[b] tokens.  Its nq_b queries
 * are the LAST nq_b tokens of that history, so query i of sequence b sits at
 * position p = k_len[b] - nq_b + i and sees keys 0..p (causal and
 * self-inclusive, [G] Stage 1: s <= t):  n_t = p + 1 candidates.
 *   prefill: B = 1, nq = k_len = L (row t sees t + 1 keys);
 *   decode:  nq_b = 1, the query sees its whole history (n = k_len[b]).
 * Precondition: 0 <= nq_b <= k_len[b].
 */
#ifndef LIBDSA_H
#define LIBDSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, inconsistent args */
  DSA_ERR_UNSUPPORTED = 2,        /* valid, but no kernel for this shape/dtype */
  DSA_ERR_WORKSPACE_TOO_SMALL = 3,
  DSA_ERR_HIP = 4                 /* a HIP launch or runtime call failed */
} dsa_status_t;

typedef enum {
  DSA_F32 = 0,        /* IEEE binary32 */
  DSA_BF16 = 1,       /* bfloat16 */
  DSA_FP8_E4M3 = 2    /* OCP FP8 E4M3 (bias 7, max 448, 0x7F/0xFF NaN) + fp32 per-token scale */
} dsa_dtype_t;

/* Ragged batch of query rows.  Arrays are device memory. */
typedef struct {
  int32_t num_seqs;             /* B >= 1 */
  int32_t num_queries;          /* T = q_seq_start[B] (host copy of that value) */
  const int32_t *q_seq_start;   /* [B+1], q_seq_start[0] = 0, non-decreasing */
  const int32_t *k_len;         /* [B], history length of each sequence */
  int32_t max_q_per_seq;        /* host bound: >= every nq_b */
  int32_t max_k_len;            /* host bound: >= every k_len[b] */
} dsa_batch_t;

/* Where a sequence's key rows live (indexer keys and latent cache alike). */
typedef struct {
  int32_t paged;                /* 0: contiguous, 1: paged */
  /* contiguous: key s of sequence b is row k_seq_start[b] + s of a
     [num_rows, width] array */
  const int64_t *k_seq_start;   /* [B] device; ignored when paged */
  /* paged: key s of sequence b is slot s % page_size of physical page
     page_table[b * page_table_stride + s / page_size] of a
     [num_rows(pages), page_size, width] pool ([P] section 4.1) */
  const int32_t *page_table;    /* [B, page_table_stride] device; ignored when contiguous */
  int32_t page_table_stride;
  int32_t page_size;            /* tokens per page; 64 is the supported value */
  int64_t num_rows;             /* contiguous: rows in the cache; paged: pages in the pool */
} dsa_kv_layout_t;

/* ------------------------------------------------------------------------
 * Stage 1: lightning-indexer scores ([G] Stage 1, ReLU score equation, in
 * its multi-head weighted form).  For every query row t and s < n_t:
 *
 *   scores[t*ld_scores + s] = scale * sq[t] * sk[s] *
 *                             sum_{j<h_i} w[t*h_i+j] * ReLU(sum_{d<d_i} q[t,j,d] * k[s,d])
 *
 * where sq / sk are the per-token FP8 scales (1 for DSA_F32).  Because the
 * scales are positive they factor out of the ReLU, so this equals the score
 * of the dequantised operands.  The [T, n, h_i] per-head products are never
 * stored.  Entries s >= n_t of each row are left untouched.
 *   dtype   DSA_FP8_E4M3 (q_idx/k_idx are bytes, q_scale/k_scale required,
 *           h_i 32, 64 or 128, d_i == 128) or DSA_F32 (scales must be NULL;
 *           h_i <= 64, d_i <= 128).
 *   q_idx   [T, h_i, d_i];  q_scale [T];  w [T, h_i] fp32
 *   k_idx   contiguous [num_rows, d_i] or paged [pages, page_size, d_i];
 *   k_scale contiguous [num_rows] or paged [pages, page_size]
 *   scale   multiplies every score (1.0, or 1/sqrt(d_i) for the page form)
 *   scores  [T, ld_scores] fp32, ld_scores >= max n_t (= max_k_len suffices)
 * ---------------------------------------------------------------------- */
dsa_status_t dsa_indexer_scores(const dsa_batch_t *batch, const dsa_kv_layout_t *keys,
                                dsa_dtype_t dtype, int32_t h_i, int32_t d_i,
                                const void *q_idx, const float *q_scale, const float *w,
                                const void *k_idx, const float *k_scale, float scale,
                                float *scores, int64_t ld_scores, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Stage 2: top-k ([G] Stage 2, TopK equation; "End-to-End Implementation"
 * for min(k, n) and ascending order).  For every query row t, writes the
 * positions of the m = min(k, n_t) largest of scores[t, 0..n_t-1] to
 * indices[t*k .. t*k+m-1] in ascending order and -1 to the remaining k - m
 * slots.  Ties go to the lowest position; scores compare by value (-0 == +0).
 * NaN scores are a precondition violation (the result is then unspecified
 * but stays in range).  The result is deterministic.
 *   1 <= k <= 65536.  workspace: dsa_topk_workspace_size() bytes, 256-byte
 *   aligned: nonzero for batches of fewer than 256 rows with histories past
 *   32768, which are selected in two passes (each 32768-long part of a row,
 *   then the union of the parts' winners) through per-row candidate lists
 *   of at most max_k_len positions and scores; 0 otherwise.
 *   DSA_ERR_WORKSPACE_TOO_SMALL if it is short.
 * ---------------------------------------------------------------------- */
dsa_status_t dsa_topk(const dsa_batch_t *batch, const float *scores, int64_t ld_scores,
                      int32_t k, int32_t *indices,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

dsa_status_t dsa_topk_workspace_size(const dsa_batch_t *batch, int32_t k, size_t *bytes);

/* ------------------------------------------------------------------------
 * Stages 1 + 2 fused: the indices dsa_topk would write for the scores
 * dsa_indexer_scores would write, without materialising the [T, n] score
 * array where a fused kernel exists.  The top-k of a row is the top-k of the
 * union of any partition of its keys, because every score depends on one key
 * only ([G] Stage 1, item 3); the fused kernel streams each row's keys in
 * ascending position and keeps a bounded list of candidates above a running
 * threshold, selecting from it exactly (same ties, same order, -1 padding).
 * It applies to FP8 keys with h_i of 32, 64 or 128 and d_i == 128 in a contiguous
 * cache, or in a paged one when max_k_len <= 131072 (each workgroup keeps
 * the page numbers of its sequence's history in LDS), for batches with
 * max_q_per_seq >= 8 (prefill, chunked prefill);
 * its workspace holds 3*k + 128 candidates (rounded up to 64) of 8 bytes
 * per query row.  Other shapes run the two stages with the fp32 score rows in
 * the workspace, followed by dsa_topk's own workspace when it needs one.
 * Arguments as for the two stages; workspace 256-byte
 * aligned, dsa_indexer_topk_workspace_size() bytes.
 * ---------------------------------------------------------------------- */
dsa_status_t dsa_indexer_topk(const dsa_batch_t *batch, const dsa_kv_layout_t *keys,
                              dsa_dtype_t dtype, int32_t h_i, int32_t d_i,
                              const void *q_idx, const float *q_scale, const float *w,
                              const void *k_idx, const float *k_scale, float scale,
                              int32_t k, int32_t *indices,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

dsa_status_t dsa_indexer_topk_workspace_size(const dsa_batch_t *batch, const dsa_kv_layout_t *keys,
                                             dsa_dtype_t dtype, int32_t h_i, int32_t d_i, int32_t k,
                                             size_t *bytes);

/* ------------------------------------------------------------------------
 * Stage 3: sparse MLA, absorbed (MQA) form ([G] Stage 2, gather and u_t
 * equations; logit of the classical MLA section).  For query row t and head
 * h, with J = { indices[t*k + j] : j < k, indices[t*k + j] >= 0 }:
 *
 *   z_s      = sm_scale * sum_{d<d_qk} q[t,h,d] * kv[s,d]        (s in J)
 *   out[t,h] = sum_s softmax_J(z)_s * kv[s, 0..d_v-1]
 *   lse[t,h] = log sum_s exp(z_s)                                (natural log)
 *
 * The key row of a token is [c^KV (d_v) ; k^R (d_qk - d_v)]: one row shared
 * by every head; the value is its first d_v entries.  An empty J gives
 * out = 0 and lse = -inf.  Indices are positions within the query's
 * sequence (as written by dsa_topk) and must be < n_t.
 *   dtype  DSA_BF16 (q, kv, out bf16; heads 16, 32, 64 or 128, d_qk == 576,
 *          d_v == 512) or DSA_F32 (heads <= 64, d_qk <= 256, d_v <= d_qk).
 *   q      [T, heads, d_qk];  kv contiguous [num_rows, d_qk] or paged
 *          [pages, page_size, d_qk];  indices [T, k] int32
 *   out    [T, heads, d_v] (dtype);  lse [T, heads] fp32, may be NULL
 *   workspace: dsa_sparse_mla_workspace_size() bytes, 16-byte aligned:
 *          the partials of rows whose selection is split over several
 *          workgroups when there are too few rows to fill the GPU (either
 *          dtype); 0 when no row is split.
 * ---------------------------------------------------------------------- */
dsa_status_t dsa_sparse_mla_fwd(const dsa_batch_t *batch, const dsa_kv_layout_t *kv_layout,
                                dsa_dtype_t dtype, int32_t heads, int32_t d_qk, int32_t d_v,
                                const void *q, const void *kv, const int32_t *indices,
                                int32_t k, float sm_scale, void *out, float *lse,
                                void *workspace, size_t workspace_bytes, hipStream_t stream);

dsa_status_t dsa_sparse_mla_workspace_size(const dsa_batch_t *batch, dsa_dtype_t dtype,
                                           int32_t heads, int32_t d_qk, int32_t d_v,
                                           int32_t k, size_t *bytes);

/* ------------------------------------------------------------------------
 * The whole path: indexer -> top-k -> sparse MLA, in the order of [G]'s
 * pipeline figure, enqueued back to back on one stream.  Both caches use the
 * same layout descriptor.  `scores` / `indices` may be NULL, in which case
 * they live in the workspace; otherwise the caller keeps them.  With
 * `scores` NULL, shapes dsa_indexer_topk fuses take the fused kernel, and no
 * score array exists at all.
 * ---------------------------------------------------------------------- */
typedef struct {
  dsa_batch_t batch;
  dsa_kv_layout_t layout;
  /* indexer */
  dsa_dtype_t index_dtype;
  int32_t h_i, d_i;
  const void *q_idx;
  const float *q_scale;
  const float *w;
  const void *k_idx;
  const float *k_scale;
  float index_scale;
  /* selection */
  int32_t top_k;
  float *scores;              /* [T, ld_scores] or NULL */
  int64_t ld_scores;          /* used when scores != NULL */
  int32_t *indices;           /* [T, top_k] or NULL */
  /* attention */
  dsa_dtype_t mla_dtype;
  int32_t heads, d_qk, d_v;
  const void *q;
  const void *kv;
  float sm_scale;
  void *out;
  float *lse;                 /* may be NULL */
} dsa_forward_args_t;

dsa_status_t dsa_forward(const dsa_forward_args_t *args, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

dsa_status_t dsa_forward_workspace_size(const dsa_forward_args_t *args, size_t *bytes);

/* ------------------------------------------------------------------------
 * dsa_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops or
 * harnesses that forbid hipMalloc.  It allocates nothing.  The workspace
 * dsa_forward would take lives in a static device array of
 * DSA_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held from
 * the library's first use on that GPU to the end of the process.
 *   args     as for dsa_forward (same validation, same results)
 *   stream   the launch stream; the array of the stream's device is used
 * Errors: DSA_ERR_WORKSPACE_TOO_SMALL, with nothing launched, when
 * dsa_forward_workspace_size(args) exceeds DSA_NOALLOC_SCRATCH_BYTES (the
 * decode workloads need 36 MiB at 32 x 32768 and 68 MiB at 64 histories of
 * up to 131072 tokens; prefill needs far more unless the caller keeps scores
 * and indices in its own buffers); otherwise as dsa_forward.
 * All calls on one GPU share its array: calls on one GPU that may overlap in
 * time (concurrent streams, or threads) race on it and must be serialised by
 * the caller.  Consecutive calls on one stream are ordered and safe.
 * ---------------------------------------------------------------------- */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)

dsa_status_t dsa_forward_noalloc(const dsa_forward_args_t *args, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Decode-step cache append.  Writes the cache entries of `num_tokens` new
 * tokens into the pools the stages above read: the FP8 indexer key with its
 * per-token scale ([G] Stage 1, item 1: the indexer's states are FP8) and
 * the latent row the sparse stage gathers ([G] Stage 2).  "Sparse Attention
 * Architectures for Long-Context Inference: Evolution and Engineering
 * Practices", section 6, names this per-step cache update.  Token i belongs
 * to sequence seq[i] at logical position pos[i]; its row is found with the
 * rules of dsa_kv_layout_t (paged: page_table[seq * stride + pos / 64],
 * slot pos % 64; contiguous: k_seq_start[seq] + pos).  In fp32:
 *
 *   amax = max_d |k_new[i,d]|;   sc = amax / 448  (1 when amax == 0)
 *   k_pool[row, d]   = E4M3 code of clamp(k_new[i,d] / sc, -448, 448),
 *                      rounded to nearest, ties to even (sign kept for zero)
 *   k_scale_pool[row] = sc
 *   latent_pool[row, :] = latent_new[i, :]    (bf16, copied bit for bit)
 *
 * Only the addressed rows are written.  Two tokens of one call must not
 * address the same row (they would race).
 *   num_tokens >= 0;  seq, pos [num_tokens] int32
 *   d_i: multiple of 4, 4..512;  k_new [num_tokens, d_i] fp32 (16-byte
 *        aligned);  k_pool contiguous [num_rows, d_i] or paged
 *        [pages, page_size, d_i] E4M3 bytes (4-byte aligned);
 *        k_scale_pool [num_rows] or [pages, page_size] fp32
 *   d_c: multiple of 8 up to 4096, or 0 for keys only (the latent pointers
 *        are then ignored);  latent_new [num_tokens, d_c] and latent_pool
 *        [num_rows, d_c] / [pages, page_size, d_c] bf16, 16-byte aligned
 *   Device-side preconditions (not checked): seq[i] is a sequence of the
 *   layout, pos[i] maps to an assigned page (paged) or a row < num_rows.
 * ---------------------------------------------------------------------- */
dsa_status_t dsa_cache_append(const dsa_kv_layout_t *layout, int32_t num_tokens,
                              const int32_t *seq, const int32_t *pos, int32_t d_i,
                              const float *k_new, void *k_pool, float *k_scale_pool,
                              int32_t d_c, const void *latent_new, void *latent_pool,
                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * The page's complete DSA module ([G] "End-to-End Implementation": the
 * DeepSeekSparseAttention module with its LightningIndexer), fp32, one query
 * token per batch element over a history of seq_len tokens:
 *
 *   k_I[b, s] = hist[b, s] . w_ki^T;   q_I[b] = q_hidden[b] . w_qi^T
 *   I[b, s]   = ReLU(q_I[b] . k_I[b, s]) / sqrt(index_dim)
 *   indices[b] = the min(top_k, seq_len) best s, ascending (ties: lowest s), -1 padded
 *   per head h: o_h = softmax_s(q_h . K_h[s] / sqrt(head_dim)) . V_h[s] over the
 *               selection, with q = q_hidden . w_q^T, K = c . w_uk^T, V = c . w_uv^T,
 *               c = latent[b, s]
 *   out[b]   = concat_h o_h . w_out^T
 *
 * The page projects every history row to k_I and decompresses K and V per
 * selected token; this computes the same function with each weight folded
 * into the side that has one vector per batch element: I[b, s] =
 * ReLU(hist[b, s] . (w_ki^T q_I[b])) / sqrt(index_dim), W_UK folded into the
 * query and W_UV applied after the softmax (matrix-vector kernels, the
 * top-k and the fp32 sparse-MLA kernels; no GEMM library).
 *   q_hidden [batch, hidden] (hidden <= 16384); hist [batch, seq_len, hidden];
 *   latent [batch, seq_len, latent_dim] (<= 256); w_qi, w_ki [index_dim, hidden];
 *   w_q, w_uk, w_uv [heads * head_dim, hidden | latent_dim] (heads <= 64);
 *   w_out [hidden, heads * head_dim]; out [batch, hidden] (batch <= 65535);
 *   indices [batch, top_k] int32.  All fp32 except indices.
 *   workspace: 256-byte aligned, dsa_module_forward_workspace_size() bytes.
 * Errors: DSA_ERR_INVALID_ARGUMENT (a size < 1, top_k outside [1, 65536], a
 * NULL tensor, an unaligned workspace), DSA_ERR_UNSUPPORTED (limits above),
 * DSA_ERR_WORKSPACE_TOO_SMALL, DSA_ERR_HIP (a launch failed); nothing is
 * enqueued when an argument is rejected.
 * ---------------------------------------------------------------------- */
dsa_status_t dsa_module_forward(int32_t batch, int32_t seq_len, int32_t hidden, int32_t heads,
                                int32_t head_dim, int32_t latent_dim, int32_t index_dim,
                                int32_t top_k, const float *q_hidden, const float *hist,
                                const float *latent, const float *w_qi, const float *w_ki,
                                const float *w_q, const float *w_uk, const float *w_uv,
                                const float *w_out, float *out, int32_t *indices,
                                void *workspace, size_t workspace_bytes, hipStream_t stream);

dsa_status_t dsa_module_forward_workspace_size(int32_t batch, int32_t seq_len, int32_t hidden,
                                               int32_t heads, int32_t head_dim,
                                               int32_t latent_dim, int32_t index_dim,
                                               size_t *bytes);

/* ------------------------------------------------------------------------
 * Precondition check on request.  The entry points above validate their
 * arguments on the host but document, without testing while they run, the
 * preconditions on device data (one read of each would cost a launch-wide
 * pass).  dsa_validate tests them on the stream, reading only, and writes
 * the first violation it finds to `report` (4 device int32):
 *   report[0] = dsa_check_code_t (0: none found);
 *   report[1..3] = where, by code:
 *     DSA_CHECK_BATCH     sequence b, its query count, k_len[b]: q_seq_start
 *                         must start at 0, not decrease, end at num_queries,
 *                         with every count <= max_q_per_seq and
 *                         count <= k_len[b] <= max_k_len;
 *     DSA_CHECK_ROWS      sequence b, k_len[b], k_seq_start[b]: a contiguous
 *                         sequence's rows must lie in [0, num_rows);
 *     DSA_CHECK_PAGE      sequence b, page index p, page id: every page a
 *                         sequence uses must be in [0, num_rows(pages));
 *     DSA_CHECK_INDEX     row t, slot j, value: indices must be -1 or in
 *                         [0, n_t) (dsa_sparse_mla_fwd's input);
 *     DSA_CHECK_NAN_SCORE row t, position s, 0: scores[t, s < n_t] must not be
 *                         NaN (dsa_topk's input).
 * The batch and layout checks always run (layout may be NULL: no row or page
 * checks); `indices` (with k) and `scores` (with ld_scores >= max_k_len) are
 * optional.  Host-side argument errors return as elsewhere and enqueue
 * nothing.  The report is valid once the stream reaches this call's end; the
 * caller reads it back.
 * ---------------------------------------------------------------------- */
typedef enum {
  DSA_CHECK_OK = 0,
  DSA_CHECK_BATCH = 1,
  DSA_CHECK_ROWS = 2,
  DSA_CHECK_PAGE = 3,
  DSA_CHECK_INDEX = 4,
  DSA_CHECK_NAN_SCORE = 5
} dsa_check_code_t;

dsa_status_t dsa_validate(const dsa_batch_t *batch, const dsa_kv_layout_t *layout,
                          const int32_t *indices, int32_t k, const float *scores,
                          int64_t ld_scores, int32_t *report, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Diagnostics.
 * ---------------------------------------------------------------------- */
const char *dsa_status_string(dsa_status_t status);   /* static string */
const char *dsa_last_error(void);   /* detail of this thread's last failure, "" if none */
int32_t dsa_abi_version(void);      /* == DSA_ABI_VERSION */

#ifdef __cplusplus
}
#endif

#endif /* LIBDSA_H */
