// Output projections after sparse MLA: the two dense bf16 GEMMs of the u_t
// equation ("DeepSeek Sparse Attention DSA Architecture Guide", "Stage 2:
// Fine-Grained Token Selection"; the implementation section's w_uv / w_out
// linear layers).  These are plain GEMMs, so they run in hipBLASLt (fp32
// accumulation): the per-head value up-projection as one strided batched
// GEMM over the heads, then the output projection.  Weights are in the
// linear-layer layout [out_features, in_features], i.e. both operands of
// every product have their reduction dimension contiguous.
//
// hipBLASLt is column-major.  A row-major [rows x cols] matrix with row
// stride ld is the column-major [cols x rows] matrix with the same ld, so the
// row-major product  Y[T x N] = X[T x K] . W[N x K]^T  is the column-major
// Y' [N x T] = W'^T [N x K] . X' [K x T]  with W' = W stored [K x N]:
// transa = T, transb = N, m = N, n = T, k = K.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "libdsa.h"

namespace {

constexpr size_t kBlasWorkspace = 32u << 20;  // library workspace carved after the intermediate

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t y_bytes(int32_t num_queries, int32_t heads, int32_t d_h) {
  return round_up((size_t)num_queries * heads * d_h * 2, 256);
}

// D (m x n) = op(A) . B (k x n), column-major, `batch` strided matrices,
// fp32 accumulation; op(A) = A^T with A stored k x m (trans_a) or A stored
// m x k.  dt: HIP_R_16BF or HIP_R_32F for every matrix.  Returns a
// description of the first failure, or nullptr.
const char *gemm(hipblasLtHandle_t h, hipDataType dt, bool trans_a, int m, int n, int k, const void *A,
                 int64_t lda, int64_t sa, const void *B, int64_t ldb, int64_t sb, void *D, int64_t ldd, int64_t sd,
                 int batch, void *ws, size_t ws_bytes, hipStream_t stream) {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  const char *err = nullptr;
  const hipblasOperation_t ta = trans_a ? HIPBLAS_OP_T : HIPBLAS_OP_N, tb = HIPBLAS_OP_N;
  const uint64_t wsb = ws_bytes;
  hipblasLtMatmulHeuristicResult_t heur{};
  int found = 0;
  const float alpha = 1.f, beta = 0.f;
  if (hipblasLtMatmulDescCreate(&desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) {
    err = "matmul descriptor";
    goto done;
  }
  hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof ta);
  hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof tb);
  if (hipblasLtMatrixLayoutCreate(&la, dt, trans_a ? k : m, trans_a ? m : k, lda) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&lb, dt, k, n, ldb) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&ld, dt, m, n, ldd) != HIPBLAS_STATUS_SUCCESS) {
    err = "matrix layouts";
    goto done;
  }
  if (batch > 1) {
    const int32_t bc = batch;
    hipblasLtMatrixLayoutSetAttribute(la, HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &bc, sizeof bc);
    hipblasLtMatrixLayoutSetAttribute(lb, HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &bc, sizeof bc);
    hipblasLtMatrixLayoutSetAttribute(ld, HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &bc, sizeof bc);
    hipblasLtMatrixLayoutSetAttribute(la, HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET, &sa, sizeof sa);
    hipblasLtMatrixLayoutSetAttribute(lb, HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET, &sb, sizeof sb);
    hipblasLtMatrixLayoutSetAttribute(ld, HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET, &sd, sizeof sd);
  }
  if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) {
    err = "preference";
    goto done;
  }
  hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof wsb);
  if (hipblasLtMatmulAlgoGetHeuristic(h, desc, la, lb, ld, ld, pref, 1, &heur, &found) != HIPBLAS_STATUS_SUCCESS ||
      found < 1) {
    err = "no hipBLASLt algorithm for this shape";
    goto done;
  }
  if (hipblasLtMatmul(h, desc, &alpha, A, la, B, lb, &beta, D, ld, D, ld, &heur.algo, ws, ws_bytes, stream) !=
      HIPBLAS_STATUS_SUCCESS)
    err = "hipblasLtMatmul";
done:
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (ld) hipblasLtMatrixLayoutDestroy(ld);
  if (lb) hipblasLtMatrixLayoutDestroy(lb);
  if (la) hipblasLtMatrixLayoutDestroy(la);
  if (desc) hipblasLtMatmulDescDestroy(desc);
  return err;
}

}  // namespace

namespace dsa {
// status and message helpers of libdsa.cpp
dsa_status_t report(dsa_status_t st, const char *fmt, ...);
}  // namespace dsa

extern "C" {

dsa_status_t dsa_blaslt_create(void **handle) {
  if (!handle) return dsa::report(DSA_ERR_INVALID_ARGUMENT, "handle is NULL");
  hipblasLtHandle_t h = nullptr;
  if (hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS) return dsa::report(DSA_ERR_HIP, "hipblasLtCreate failed");
  *handle = (void *)h;
  return dsa::report(DSA_OK, "");
}

dsa_status_t dsa_blaslt_destroy(void *handle) {
  if (handle && hipblasLtDestroy((hipblasLtHandle_t)handle) != HIPBLAS_STATUS_SUCCESS)
    return dsa::report(DSA_ERR_HIP, "hipblasLtDestroy failed");
  return dsa::report(DSA_OK, "");
}

dsa_status_t dsa_output_projection_workspace_size(int32_t num_queries, int32_t heads, int32_t d_h, size_t *bytes) {
  if (!bytes) return dsa::report(DSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (num_queries < 0 || heads < 1 || d_h < 1)
    return dsa::report(DSA_ERR_INVALID_ARGUMENT, "output projection: num_queries >= 0, heads >= 1, d_h >= 1");
  *bytes = y_bytes(num_queries, heads, d_h) + kBlasWorkspace;
  return dsa::report(DSA_OK, "");
}

dsa_status_t dsa_output_projection(void *blaslt, int32_t num_queries, int32_t heads, int32_t d_c, int32_t d_h,
                                   int32_t hidden, const void *o, const void *w_uv, const void *w_o, void *out,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!blaslt) return dsa::report(DSA_ERR_INVALID_ARGUMENT, "output projection: hipBLASLt handle is NULL");
  if (num_queries < 0 || heads < 1 || d_c < 1 || d_h < 1 || hidden < 1)
    return dsa::report(DSA_ERR_INVALID_ARGUMENT, "output projection: sizes must be positive (num_queries >= 0)");
  if (d_c % 8 || d_h % 8 || hidden % 8)
    return dsa::report(DSA_ERR_UNSUPPORTED, "output projection: d_c, d_h and hidden must be multiples of 8");
  const size_t need = y_bytes(num_queries, heads, d_h) + kBlasWorkspace;
  if (workspace_bytes < need || !workspace)
    return dsa::report(DSA_ERR_WORKSPACE_TOO_SMALL, "output projection needs %zu workspace bytes, got %zu", need,
                       workspace_bytes);
  if ((uintptr_t)workspace % 256) return dsa::report(DSA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (num_queries == 0) return dsa::report(DSA_OK, "");
  if (!o || !w_uv || !w_o || !out)
    return dsa::report(DSA_ERR_INVALID_ARGUMENT, "output projection: o, w_uv, w_o and out must be non-NULL");
  auto h = (hipblasLtHandle_t)blaslt;
  void *y = workspace;
  void *ws = (char *)workspace + y_bytes(num_queries, heads, d_h);
  const int T = num_queries;
  // y[t, h, :] = W_UV,h . o[t, h, :]: per head m = d_h, n = T, k = d_c
  const char *err = gemm(h, HIP_R_16BF, true, d_h, T, d_c, w_uv, d_c, (int64_t)d_h * d_c, o, (int64_t)heads * d_c,
                         d_c, y, (int64_t)heads * d_h, d_h, heads, ws, kBlasWorkspace, stream);
  if (err) return dsa::report(DSA_ERR_HIP, "output projection, W_UV: %s", err);
  // out[t, :] = W_O . y[t, :]: m = hidden, n = T, k = heads * d_h
  const int K = heads * d_h;
  err = gemm(h, HIP_R_16BF, true, hidden, T, K, w_o, K, 0, y, K, 0, out, hidden, 0, 1, ws, kBlasWorkspace, stream);
  if (err) return dsa::report(DSA_ERR_HIP, "output projection, W_O: %s", err);
  return dsa::report(DSA_OK, "");
}

}  // extern "C"

// ------------------------------------------------------------------------
// The page's complete DSA module ("DeepSeek Sparse Attention DSA Architecture
// Guide", "End-to-End Implementation": DeepSeekSparseAttention with its
// LightningIndexer), fp32, one query token per batch element over an S-token
// history.  The page decompresses every selected latent row into per-head
// keys and values (W_UK, W_UV); here W_UK is folded into the query and W_UV
// applied after the softmax, the same function with (hidden-size) GEMMs in
// place of per-token decompressions:
//   k_I = hist . W_kI^T,  q_I = h_q . W_qI^T            (hipBLASLt)
//   scores, top-k                                        (indexer and top-k kernels)
//   q = h_q . W_Q^T;  q_abs[h] = W_UK,h^T q[h]           (hipBLASLt, batched over heads)
//   o_abs[h] = softmax_S(q_abs[h] . c_s / sqrt(d_h)) . c_s    (fp32 sparse MLA kernel)
//   y[h] = W_UV,h o_abs[h];  out = y . W_out^T           (hipBLASLt)
// ------------------------------------------------------------------------
namespace dsa {
size_t mla_f32_workspace_bound(int num_queries, int heads, int d_v);
}  // namespace dsa

namespace {
struct ModuleWs {
  size_t meta, k_idx, q_idx, scores, q, q_abs, o_abs, y, mla, mla_bytes, blas, total;
  int64_t ld;
};

ModuleWs module_ws(int32_t B, int32_t S, int32_t H, int32_t d_h, int32_t d_c, int32_t d_i) {
  ModuleWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += round_up(bytes, 256); return at; };
  w.ld = (int64_t)round_up((size_t)S, 4);
  w.meta = take(((size_t)B + 1) * 4 + (size_t)B * 4 + (size_t)B * 8 + (size_t)B * 4 + 64);
  w.k_idx = take((size_t)B * S * d_i * 4);
  w.q_idx = take((size_t)B * d_i * 4);
  w.scores = take((size_t)B * w.ld * 4);
  w.q = take((size_t)B * H * d_h * 4);
  w.q_abs = take((size_t)B * H * d_c * 4);
  w.o_abs = take((size_t)B * H * d_c * 4);
  w.y = take((size_t)B * H * d_h * 4);
  w.mla_bytes = dsa::mla_f32_workspace_bound(B, H, d_c);
  w.mla = take(w.mla_bytes);
  w.blas = take(kBlasWorkspace);
  w.total = off;
  return w;
}
}  // namespace

namespace dsa {
hipError_t launch_module_meta(int batch, int seq_len, int32_t *q_seq_start, int32_t *k_len, int64_t *k_seq_start,
                              float *ones, hipStream_t stream);
}  // namespace dsa

extern "C" {

dsa_status_t dsa_module_forward_workspace_size(int32_t batch, int32_t seq_len, int32_t heads, int32_t head_dim,
                                               int32_t latent_dim, int32_t index_dim, size_t *bytes) {
  if (!bytes) return dsa::report(DSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (batch < 1 || seq_len < 1 || heads < 1 || head_dim < 1 || latent_dim < 1 || index_dim < 1)
    return dsa::report(DSA_ERR_INVALID_ARGUMENT, "module forward: every size must be >= 1");
  *bytes = module_ws(batch, seq_len, heads, head_dim, latent_dim, index_dim).total;
  return dsa::report(DSA_OK, "");
}

dsa_status_t dsa_module_forward(void *blaslt, int32_t batch, int32_t seq_len, int32_t hidden, int32_t heads,
                                int32_t head_dim, int32_t latent_dim, int32_t index_dim, int32_t top_k,
                                const float *q_hidden, const float *hist, const float *latent, const float *w_qi,
                                const float *w_ki, const float *w_q, const float *w_uk, const float *w_uv,
                                const float *w_out, float *out, int32_t *indices, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  if (!blaslt) return dsa::report(DSA_ERR_INVALID_ARGUMENT, "module forward: hipBLASLt handle is NULL");
  if (batch < 1 || seq_len < 1 || hidden < 1 || heads < 1 || head_dim < 1 || latent_dim < 1 || index_dim < 1)
    return dsa::report(DSA_ERR_INVALID_ARGUMENT, "module forward: every size must be >= 1");
  if (heads > 64 || latent_dim > 256 || index_dim > 128)
    return dsa::report(DSA_ERR_UNSUPPORTED, "module forward: needs heads <= 64, latent_dim <= 256, index_dim <= 128");
  if (top_k < 1 || top_k > 65536) return dsa::report(DSA_ERR_INVALID_ARGUMENT, "module forward: top_k in [1, 65536]");
  if ((int64_t)batch * seq_len > INT32_MAX)
    return dsa::report(DSA_ERR_UNSUPPORTED, "module forward: batch * seq_len must fit in int32");
  if (!q_hidden || !hist || !latent || !w_qi || !w_ki || !w_q || !w_uk || !w_uv || !w_out || !out || !indices)
    return dsa::report(DSA_ERR_INVALID_ARGUMENT, "module forward: a tensor pointer is NULL");
  const ModuleWs w = module_ws(batch, seq_len, heads, head_dim, latent_dim, index_dim);
  if (workspace_bytes < w.total || !workspace)
    return dsa::report(DSA_ERR_WORKSPACE_TOO_SMALL, "module forward needs %zu workspace bytes, got %zu", w.total,
                       workspace_bytes);
  if ((uintptr_t)workspace % 256) return dsa::report(DSA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  char *base = (char *)workspace;
  auto h = (hipblasLtHandle_t)blaslt;
  const int B = batch, S = seq_len, H = heads, d_h = head_dim, d_c = latent_dim, d_i = index_dim;
  int32_t *q_seq_start = (int32_t *)(base + w.meta);
  int32_t *k_len = q_seq_start + (B + 1);
  int64_t *k_seq_start = (int64_t *)(((uintptr_t)(k_len + B) + 7) / 8 * 8);
  float *ones = (float *)(k_seq_start + B);
  float *k_idx = (float *)(base + w.k_idx), *q_idx = (float *)(base + w.q_idx), *scores = (float *)(base + w.scores);
  float *q = (float *)(base + w.q), *q_abs = (float *)(base + w.q_abs), *o_abs = (float *)(base + w.o_abs);
  float *y = (float *)(base + w.y);
  void *bws = base + w.blas;
  hipError_t e = dsa::launch_module_meta(B, S, q_seq_start, k_len, k_seq_start, ones, stream);
  if (e != hipSuccess) return dsa::report(DSA_ERR_HIP, "module forward: batch arrays: %s", hipGetErrorString(e));
  const char *err;
  // indexer keys and query: k_I = hist . W_kI^T (B*S rows), q_I = h_q . W_qI^T
  if ((err = gemm(h, HIP_R_32F, true, d_i, B * S, hidden, w_ki, hidden, 0, hist, hidden, 0, k_idx, d_i, 0, 1, bws,
                  kBlasWorkspace, stream)))
    return dsa::report(DSA_ERR_HIP, "module forward, indexer keys: %s", err);
  if ((err = gemm(h, HIP_R_32F, true, d_i, B, hidden, w_qi, hidden, 0, q_hidden, hidden, 0, q_idx, d_i, 0, 1, bws,
                  kBlasWorkspace, stream)))
    return dsa::report(DSA_ERR_HIP, "module forward, indexer query: %s", err);
  // scores (one head, weight 1, scale 1/sqrt(d_I)) and top-k over each full history
  const dsa_batch_t bt{B, B, q_seq_start, k_len, 1, S};
  const dsa_kv_layout_t ly{0, k_seq_start, nullptr, 0, 64, (int64_t)B * S};
  dsa_status_t st = dsa_indexer_scores(&bt, &ly, DSA_F32, 1, d_i, q_idx, nullptr, ones, k_idx, nullptr,
                                       1.f / sqrtf((float)d_i), scores, w.ld, stream);
  if (st != DSA_OK) return st;
  st = dsa_topk(&bt, scores, w.ld, top_k, indices, nullptr, 0, stream);
  if (st != DSA_OK) return st;
  // q = h_q . W_Q^T; q_abs[b, h, :] = W_UK,h^T q[b, h, :] (W_UK,h stored d_h x d_c)
  if ((err = gemm(h, HIP_R_32F, true, H * d_h, B, hidden, w_q, hidden, 0, q_hidden, hidden, 0, q, H * d_h, 0, 1,
                  bws, kBlasWorkspace, stream)))
    return dsa::report(DSA_ERR_HIP, "module forward, query: %s", err);
  if ((err = gemm(h, HIP_R_32F, false, d_c, B, d_h, w_uk, d_c, (int64_t)d_h * d_c, q, (int64_t)H * d_h, d_h, q_abs,
                  (int64_t)H * d_c, d_c, H, bws, kBlasWorkspace, stream)))
    return dsa::report(DSA_ERR_HIP, "module forward, W_UK: %s", err);
  // softmax over the selected latent rows, per head, scale 1/sqrt(d_h)
  const dsa_kv_layout_t lat_ly{0, k_seq_start, nullptr, 0, 64, (int64_t)B * S};
  st = dsa_sparse_mla_fwd(&bt, &lat_ly, DSA_F32, H, d_c, d_c, q_abs, latent, indices, top_k,
                          1.f / sqrtf((float)d_h), o_abs, nullptr, base + w.mla, w.mla_bytes, stream);
  if (st != DSA_OK) return st;
  // y[b, h, :] = W_UV,h o_abs[b, h, :]; out = y . W_out^T
  if ((err = gemm(h, HIP_R_32F, true, d_h, B, d_c, w_uv, d_c, (int64_t)d_h * d_c, o_abs, (int64_t)H * d_c, d_c, y,
                  (int64_t)H * d_h, d_h, H, bws, kBlasWorkspace, stream)))
    return dsa::report(DSA_ERR_HIP, "module forward, W_UV: %s", err);
  if ((err = gemm(h, HIP_R_32F, true, hidden, B, H * d_h, w_out, H * d_h, 0, y, H * d_h, 0, out, hidden, 0, 1, bws,
                  kBlasWorkspace, stream)))
    return dsa::report(DSA_ERR_HIP, "module forward, W_out: %s", err);
  return dsa::report(DSA_OK, "");
}

}  // extern "C"
