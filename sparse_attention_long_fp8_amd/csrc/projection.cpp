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

#include "libdsa_proj.h"

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
