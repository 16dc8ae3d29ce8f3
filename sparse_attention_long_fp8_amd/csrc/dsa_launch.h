// Internal launcher entry points of the libdsa kernels (C++ linkage; the
// public C ABI lives in include/libdsa.h and is implemented in libdsa.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct BatchDev;
struct KeysDev;

hipError_t launch_indexer_f32(const BatchDev &bt, const KeysDev &kd, int num_queries,
                              int max_k_len, int h_i, int d_i, const float *q, const float *w,
                              const float *k, float scale, float *scores, int64_t ld,
                              hipStream_t stream);

hipError_t launch_indexer_fp8(const BatchDev &bt, const KeysDev &kd, int num_seqs, int num_queries,
                              int max_q_per_seq, int max_k_len, int h_i, const uint8_t *q,
                              const float *q_scale, const float *w, const uint8_t *k,
                              const float *k_scale, float scale, float *scores, int64_t ld,
                              hipStream_t stream);

// Fused indexer -> top-k (FP8, 32, 64 or 128 heads x 128; contiguous keys, or paged
// histories of at most fused_topk_max_paged_keys keys): candidate list
// capacity per row and workspace bytes.
int fused_topk_cap(int k, int max_k_len);
size_t fused_topk_workspace_bytes(int num_queries, int k, int max_k_len);
constexpr int fused_topk_max_paged_keys = 2048 * 64;
hipError_t launch_indexer_topk_fused(const BatchDev &bt, const KeysDev &kd, int num_seqs, int num_queries,
                                     int max_q_per_seq, int max_k_len, int h_i, const uint8_t *q,
                                     const float *q_scale, const float *w, const uint8_t *k, const float *k_scale,
                                     float scale, int topk, int32_t *indices, void *workspace, hipStream_t stream);

// Top-k; batches of few rows with histories past the LDS row cache use a
// workspace of topk_workspace_bytes (0 otherwise).
size_t topk_workspace_bytes(int num_queries, int max_k_len, int k);
hipError_t launch_topk(const BatchDev &bt, int num_queries, int max_k_len, const float *scores, int64_t ld,
                       int k, int32_t *indices, void *workspace, hipStream_t stream);

// Split count the bf16 sparse-MLA kernel uses for this many query rows
// (1 = no split, no workspace).
int mla_bf16_splits(int num_queries, int heads, int k);
size_t mla_bf16_workspace_bytes(int num_queries, int heads, int d_v, int k);

// Split count and workspace of the fp32 sparse-MLA kernel (1 split = no
// workspace).
int mla_f32_splits(int num_queries, int k);
size_t mla_f32_workspace_bytes(int num_queries, int heads, int d_v, int k);
size_t mla_f32_workspace_bound(int num_queries, int heads, int d_v);  // over every k

hipError_t launch_mla_f32(const BatchDev &bt, const KeysDev &kd, int num_queries, int heads,
                          int d_qk, int d_v, const float *q, const float *kv,
                          const int32_t *indices, int k, float sm_scale, float *out, float *lse,
                          void *workspace, hipStream_t stream);

hipError_t launch_mla_bf16(const BatchDev &bt, const KeysDev &kd, int num_queries, int heads,
                           const void *q, const void *kv, const int32_t *indices, int k,
                           float sm_scale, void *out, float *lse, void *workspace,
                           hipStream_t stream);

hipError_t launch_cache_append(const KeysDev &kd, int num_tokens, const int32_t *seq,
                               const int32_t *pos, int d_i, const float *k_new, void *k_pool,
                               float *k_scale_pool, int d_c, const void *latent_new,
                               void *latent_pool, hipStream_t stream);

// On-request precondition checks (dsa_validate).  Codes match
// dsa_check_code_t in libdsa.h.
enum { kCheckBatch = 1, kCheckRows = 2, kCheckPage = 3, kCheckIndex = 4, kCheckNanScore = 5 };
struct ValidateArgs {
  int32_t num_seqs, num_queries, max_q_per_seq, max_k_len;
  const int32_t *q_seq_start, *k_len;  // NULL (empty batch): only the report is cleared
  int32_t has_layout;                  // 0: no row or page checks
  int32_t paged;
  const int64_t *k_seq_start;
  const int32_t *page_table;
  int32_t page_table_stride;
  int64_t num_rows;
  const int32_t *indices;  // [T, k] or NULL
  int32_t k;
  const float *scores;     // [T, ld] or NULL
  int64_t ld;
};
hipError_t launch_validate(const ValidateArgs &a, int32_t *report, hipStream_t stream);

// Matrix-vector products of the page-module entry point (fp32).
// Row job: y[b * y_b_stride + r] = sum_c w[r * cols + c] * x[b * x_b_stride +
// (r / rows_per_group) * x_g_stride + c] for r < rows; vec4 when cols and
// both strides are multiples of 4 and w, x are 16-byte aligned.
struct GemvRowJob {
  const float *w;
  const float *x;
  float *y;
  int rows, cols, rows_per_group, vec4;
  int64_t x_b_stride, x_g_stride, y_b_stride;
  int blocks;  // set by the launcher
};
// Column job: y[b * y_b_stride + g * y_g_stride + c] = sum_{j<J}
// w[(g * J + j) * cols + c] * x[b * x_b_stride + g * x_g_stride + j].
struct GemvColJob {
  const float *w;
  const float *x;
  float *y;
  int groups, J, cols;
  int64_t x_b_stride, x_g_stride, y_b_stride, y_g_stride;
  int blocks;  // set by the launcher
};
// Two independent jobs per launch (the second may have w == NULL).
hipError_t launch_gemv_rows(GemvRowJob j0, GemvRowJob j1, int batch, hipStream_t stream);
hipError_t launch_gemv_cols(GemvColJob j0, GemvColJob j1, int batch, hipStream_t stream);
// scores[b * ld + s] = max(hist[b, s, :] . u[b, :], 0) * scale, s < S
// (hidden <= 16384: u[b] is staged in LDS).
hipError_t launch_module_scores(const float *hist, const float *u, int batch, int S, int hidden, float scale,
                                float *scores, int64_t ld, hipStream_t stream);
hipError_t launch_module_meta(int batch, int seq_len, int32_t *q_seq_start, int32_t *k_len,
                              int64_t *k_seq_start, float *ones, hipStream_t stream);

}  // namespace dsa
