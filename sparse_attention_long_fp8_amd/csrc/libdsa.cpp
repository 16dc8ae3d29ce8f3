// libdsa host library: argument validation, workspace sizing and kernel
// dispatch behind the C ABI of include/libdsa.h.  Nothing here allocates,
// frees or synchronises; every call validates first and only then enqueues.
#include "libdsa.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "dsa_device.h"
#include "dsa_launch.h"

namespace {

thread_local std::string g_last_error;

dsa_status_t fail(dsa_status_t st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dsa_status_t ok() {
  g_last_error.clear();
  return DSA_OK;
}

dsa_status_t hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

dsa_status_t check_batch(const dsa_batch_t *bt) {
  if (!bt) return fail(DSA_ERR_INVALID_ARGUMENT, "batch is NULL");
  if (bt->num_seqs < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 1");
  if (bt->num_queries < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "num_queries must be >= 0");
  if (bt->max_q_per_seq < 0 || bt->max_k_len < 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, "max_q_per_seq / max_k_len must be >= 0");
  if (bt->max_q_per_seq > bt->max_k_len)
    return fail(DSA_ERR_INVALID_ARGUMENT, "max_q_per_seq exceeds max_k_len (queries are the last tokens of their history)");
  if (bt->num_queries > 0) {
    if (!bt->q_seq_start || !bt->k_len) return fail(DSA_ERR_INVALID_ARGUMENT, "q_seq_start / k_len is NULL");
    if (bt->max_k_len < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "max_k_len must be >= 1 when there are queries");
    if ((int64_t)bt->num_queries > (int64_t)bt->num_seqs * bt->max_q_per_seq)
      return fail(DSA_ERR_INVALID_ARGUMENT, "num_queries exceeds num_seqs * max_q_per_seq");
  }
  return DSA_OK;
}

dsa_status_t check_layout(const dsa_kv_layout_t *ly, const dsa_batch_t *bt, const char *what) {
  if (!ly) return fail(DSA_ERR_INVALID_ARGUMENT, "%s layout is NULL", what);
  if (ly->paged != 0 && ly->paged != 1) return fail(DSA_ERR_INVALID_ARGUMENT, "%s layout: paged must be 0 or 1", what);
  if (ly->num_rows < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "%s layout: num_rows must be >= 1", what);
  if (ly->paged) {
    if (!ly->page_table) return fail(DSA_ERR_INVALID_ARGUMENT, "%s layout: page_table is NULL", what);
    if (ly->page_size != dsa::kPageSize)
      return fail(DSA_ERR_UNSUPPORTED, "%s layout: page_size %d (only %d is implemented)", what, ly->page_size, dsa::kPageSize);
    const int64_t need = ((int64_t)bt->max_k_len + ly->page_size - 1) / ly->page_size;
    if (ly->page_table_stride < need)
      return fail(DSA_ERR_INVALID_ARGUMENT, "%s layout: page_table_stride %d < pages of max_k_len (%lld)", what,
                  ly->page_table_stride, (long long)need);
  } else {
    if (!ly->k_seq_start) return fail(DSA_ERR_INVALID_ARGUMENT, "%s layout: k_seq_start is NULL", what);
    if (ly->num_rows < bt->max_k_len)
      return fail(DSA_ERR_INVALID_ARGUMENT, "%s layout: num_rows %lld < max_k_len %d", what, (long long)ly->num_rows, bt->max_k_len);
  }
  return DSA_OK;
}

// A batch whose every sequence has exactly one query row (the declared counts
// allow nothing else) lets the kernels skip the sequence search.
dsa::BatchDev to_dev(const dsa_batch_t *bt) {
  const int one = bt->num_queries == bt->num_seqs && bt->max_q_per_seq == 1;
  return dsa::BatchDev{bt->num_seqs, bt->q_seq_start, bt->k_len, one};
}

dsa::KeysDev to_dev(const dsa_kv_layout_t *ly) {
  return dsa::KeysDev{ly->paged, ly->k_seq_start, ly->page_table, ly->page_table_stride};
}

dsa_status_t check_indexer(const dsa_batch_t *bt, const dsa_kv_layout_t *ly, dsa_dtype_t dt, int32_t h_i,
                           int32_t d_i, const void *q_idx, const float *q_scale, const float *w,
                           const void *k_idx, const float *k_scale, float scale, const float *scores,
                           int64_t ld) {
  dsa_status_t st = check_batch(bt);
  if (st != DSA_OK) return st;
  if ((st = check_layout(ly, bt, "key")) != DSA_OK) return st;
  if (!std::isfinite(scale)) return fail(DSA_ERR_INVALID_ARGUMENT, "indexer scale must be finite");
  if (ld < bt->max_k_len) return fail(DSA_ERR_INVALID_ARGUMENT, "ld_scores %lld < max_k_len %d", (long long)ld, bt->max_k_len);
  if (dt == DSA_FP8_E4M3) {
    if (d_i != 128) return fail(DSA_ERR_UNSUPPORTED, "FP8 indexer: d_i must be 128 (got %d)", d_i);
    if (h_i != 32 && h_i != 64 && h_i != 128) return fail(DSA_ERR_UNSUPPORTED, "FP8 indexer: h_i must be 32, 64 or 128 (got %d)", h_i);
    if (bt->num_queries > 0 && (!q_scale || !k_scale)) return fail(DSA_ERR_INVALID_ARGUMENT, "FP8 indexer needs q_scale and k_scale");
    if (!aligned(q_idx, 32) || !aligned(k_idx, 32)) return fail(DSA_ERR_INVALID_ARGUMENT, "FP8 q_idx / k_idx must be 32-byte aligned");
  } else if (dt == DSA_F32) {
    if (h_i < 1 || h_i > 64 || d_i < 1 || d_i > 128) return fail(DSA_ERR_UNSUPPORTED, "f32 indexer: needs 1 <= h_i <= 64, 1 <= d_i <= 128");
    if (q_scale || k_scale) return fail(DSA_ERR_INVALID_ARGUMENT, "f32 indexer takes no scales (pass NULL)");
  } else {
    return fail(DSA_ERR_UNSUPPORTED, "indexer dtype must be DSA_F32 or DSA_FP8_E4M3");
  }
  if (bt->num_queries > 0 && (!q_idx || !w || !k_idx || !scores))
    return fail(DSA_ERR_INVALID_ARGUMENT, "indexer: q_idx, w, k_idx and scores must be non-NULL");
  return DSA_OK;
}

dsa_status_t check_topk(const dsa_batch_t *bt, const float *scores, int64_t ld, int32_t k, const int32_t *indices) {
  dsa_status_t st = check_batch(bt);
  if (st != DSA_OK) return st;
  if (k < 1 || k > 65536) return fail(DSA_ERR_INVALID_ARGUMENT, "top-k: k must be in [1, 65536] (got %d)", k);
  if (ld < bt->max_k_len) return fail(DSA_ERR_INVALID_ARGUMENT, "ld_scores %lld < max_k_len %d", (long long)ld, bt->max_k_len);
  if (bt->num_queries > 0) {
    if (!scores || !indices) return fail(DSA_ERR_INVALID_ARGUMENT, "top-k: scores / indices is NULL");
    if (!aligned(scores, 16) || ld % 4 != 0) return fail(DSA_ERR_INVALID_ARGUMENT, "top-k: scores must be 16-byte aligned with ld_scores % 4 == 0");
  }
  return DSA_OK;
}

dsa_status_t check_mla(const dsa_batch_t *bt, const dsa_kv_layout_t *ly, dsa_dtype_t dt, int32_t heads, int32_t d_qk,
                       int32_t d_v, const void *q, const void *kv, const int32_t *indices, int32_t k, float sm_scale,
                       const void *out) {
  dsa_status_t st = check_batch(bt);
  if (st != DSA_OK) return st;
  if ((st = check_layout(ly, bt, "latent")) != DSA_OK) return st;
  if (k < 1 || k > 65536) return fail(DSA_ERR_INVALID_ARGUMENT, "sparse MLA: k must be in [1, 65536] (got %d)", k);
  if (!std::isfinite(sm_scale)) return fail(DSA_ERR_INVALID_ARGUMENT, "sm_scale must be finite");
  if (dt == DSA_BF16) {
    if (d_qk != 576 || d_v != 512) return fail(DSA_ERR_UNSUPPORTED, "bf16 sparse MLA: d_qk must be 576 and d_v 512 (got %d, %d)", d_qk, d_v);
    if (heads != 16 && heads != 32 && heads != 64 && heads != 128)
      return fail(DSA_ERR_UNSUPPORTED, "bf16 sparse MLA: heads must be 16, 32, 64 or 128 (got %d)", heads);
    if (!aligned(q, 16) || !aligned(kv, 16)) return fail(DSA_ERR_INVALID_ARGUMENT, "bf16 q / kv must be 16-byte aligned");
  } else if (dt == DSA_F32) {
    if (heads < 1 || heads > 64 || d_qk < 1 || d_qk > 256 || d_v < 1 || d_v > d_qk)
      return fail(DSA_ERR_UNSUPPORTED, "f32 sparse MLA: needs 1 <= heads <= 64, 1 <= d_v <= d_qk <= 256");
  } else {
    return fail(DSA_ERR_UNSUPPORTED, "sparse MLA dtype must be DSA_F32 or DSA_BF16");
  }
  if (bt->num_queries > 0 && (!q || !kv || !indices || !out))
    return fail(DSA_ERR_INVALID_ARGUMENT, "sparse MLA: q, kv, indices and out must be non-NULL");
  return DSA_OK;
}

size_t mla_ws(const dsa_batch_t *bt, dsa_dtype_t dt, int32_t heads, int32_t d_v, int32_t k) {
  if (dt == DSA_F32) return dsa::mla_f32_workspace_bytes(bt->num_queries, heads, d_v, k);
  if (dt != DSA_BF16) return 0;
  return dsa::mla_bf16_workspace_bytes(bt->num_queries, heads, d_v, k);
}

// The fused indexer -> top-k kernel covers FP8 keys of 32, 64 or 128 heads x
// 128 in a contiguous cache, or a paged one with histories of at most
// fused_topk_max_paged_keys keys, for batches with at least 8 query rows per
// sequence.
bool fused_applies(const dsa_batch_t *bt, const dsa_kv_layout_t *ly, dsa_dtype_t dt, int32_t h_i, int32_t d_i) {
  return dt == DSA_FP8_E4M3 && (h_i == 32 || h_i == 64 || h_i == 128) && d_i == 128 && bt->max_q_per_seq >= 8 &&
         (!ly->paged || bt->max_k_len <= dsa::fused_topk_max_paged_keys);
}

// Workspace of dsa_indexer_topk: the fused kernel's candidate lists, or the
// fp32 score rows the two separate stages pass between them.
size_t indexer_topk_ws(const dsa_batch_t *bt, const dsa_kv_layout_t *ly, dsa_dtype_t dt, int32_t h_i, int32_t d_i,
                       int32_t k) {
  if (fused_applies(bt, ly, dt, h_i, d_i)) return dsa::fused_topk_workspace_bytes(bt->num_queries, k, bt->max_k_len);
  return round_up((size_t)bt->num_queries * round_up((size_t)bt->max_k_len, 4) * sizeof(float), 256) +
         dsa::topk_workspace_bytes(bt->num_queries, bt->max_k_len, k);
}

// Workspace carve-up of dsa_forward: [scores or fused candidate lists][indices][mla partials],
// 256-byte aligned.  Without caller-kept scores, shapes the fused indexer -> top-k kernel
// covers use it, and the region holds its candidate lists instead of the score rows.
struct ForwardWs {
  int64_t ld;
  bool fused;
  size_t scores_off, indices_off, topk_off, topk_bytes, mla_off, total;
};

ForwardWs forward_ws(const dsa_forward_args_t *a) {
  ForwardWs w{};
  const size_t T = (size_t)a->batch.num_queries;
  w.ld = a->scores ? a->ld_scores : (int64_t)round_up((size_t)a->batch.max_k_len, 4);
  w.fused = !a->scores && fused_applies(&a->batch, &a->layout, a->index_dtype, a->h_i, a->d_i);
  size_t off = 0;
  w.scores_off = off;
  if (w.fused)
    off += round_up(dsa::fused_topk_workspace_bytes(a->batch.num_queries, a->top_k, a->batch.max_k_len), 256);
  else if (!a->scores)
    off += round_up(T * (size_t)w.ld * sizeof(float), 256);
  w.indices_off = off;
  if (!a->indices) off += round_up(T * (size_t)a->top_k * sizeof(int32_t), 256);
  w.topk_off = off;
  w.topk_bytes = w.fused ? 0 : dsa::topk_workspace_bytes(a->batch.num_queries, a->batch.max_k_len, a->top_k);
  off += w.topk_bytes;
  w.mla_off = off;
  off += round_up(mla_ws(&a->batch, a->mla_dtype, a->heads, a->d_v, a->top_k), 256);
  w.total = off;
  return w;
}

}  // namespace

namespace dsa {
// Status reporting for the other host sources of the library (records the
// message dsa_last_error() returns; DSA_OK clears it).
dsa_status_t report(dsa_status_t st, const char *fmt, ...) {
  if (st == DSA_OK) return ok();
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}
}  // namespace dsa

extern "C" {

int32_t dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char *dsa_status_string(dsa_status_t st) {
  switch (st) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARGUMENT: return "DSA_ERR_INVALID_ARGUMENT";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE_TOO_SMALL: return "DSA_ERR_WORKSPACE_TOO_SMALL";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "unknown dsa_status_t";
}

const char *dsa_last_error(void) { return g_last_error.c_str(); }

dsa_status_t dsa_indexer_scores(const dsa_batch_t *batch, const dsa_kv_layout_t *keys, dsa_dtype_t dtype,
                                int32_t h_i, int32_t d_i, const void *q_idx, const float *q_scale, const float *w,
                                const void *k_idx, const float *k_scale, float scale, float *scores,
                                int64_t ld_scores, hipStream_t stream) {
  dsa_status_t st = check_indexer(batch, keys, dtype, h_i, d_i, q_idx, q_scale, w, k_idx, k_scale, scale, scores,
                                  ld_scores);
  if (st != DSA_OK) return st;
  if (batch->num_queries == 0) return ok();
  const dsa::BatchDev bt = to_dev(batch);
  const dsa::KeysDev kd = to_dev(keys);
  hipError_t e;
  if (dtype == DSA_FP8_E4M3)
    e = dsa::launch_indexer_fp8(bt, kd, batch->num_seqs, batch->num_queries, batch->max_q_per_seq, batch->max_k_len,
                                h_i, (const uint8_t *)q_idx, q_scale, w, (const uint8_t *)k_idx, k_scale, scale,
                                scores, ld_scores, stream);
  else
    e = dsa::launch_indexer_f32(bt, kd, batch->num_queries, batch->max_k_len, h_i, d_i, (const float *)q_idx, w,
                                (const float *)k_idx, scale, scores, ld_scores, stream);
  return hip_status(e, "indexer launch");
}

dsa_status_t dsa_topk_workspace_size(const dsa_batch_t *batch, int32_t k, size_t *bytes) {
  if (!bytes) return fail(DSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  dsa_status_t st = check_batch(batch);
  if (st != DSA_OK) return st;
  if (k < 1 || k > 65536) return fail(DSA_ERR_INVALID_ARGUMENT, "top-k: k must be in [1, 65536] (got %d)", k);
  *bytes = dsa::topk_workspace_bytes(batch->num_queries, batch->max_k_len, k);
  return ok();
}

dsa_status_t dsa_validate(const dsa_batch_t *batch, const dsa_kv_layout_t *layout, const int32_t *indices,
                          int32_t k, const float *scores, int64_t ld_scores, int32_t *report, hipStream_t stream) {
  dsa_status_t st = check_batch(batch);
  if (st != DSA_OK) return st;
  if (layout && (st = check_layout(layout, batch, "key")) != DSA_OK) return st;
  if (!report) return fail(DSA_ERR_INVALID_ARGUMENT, "validate: report is NULL");
  if (!aligned(report, 4)) return fail(DSA_ERR_INVALID_ARGUMENT, "validate: report must be 4-byte aligned");
  if (indices && (k < 1 || k > 65536)) return fail(DSA_ERR_INVALID_ARGUMENT, "validate: k must be in [1, 65536]");
  if (scores && ld_scores < batch->max_k_len)
    return fail(DSA_ERR_INVALID_ARGUMENT, "validate: ld_scores %lld < max_k_len %d", (long long)ld_scores,
                batch->max_k_len);
  if (batch->num_queries > 0 && (!batch->q_seq_start || !batch->k_len))
    return fail(DSA_ERR_INVALID_ARGUMENT, "validate: q_seq_start / k_len is NULL");
  dsa::ValidateArgs a{};
  a.num_seqs = batch->num_seqs;
  a.num_queries = batch->num_queries;
  a.max_q_per_seq = batch->max_q_per_seq;
  a.max_k_len = batch->max_k_len;
  a.q_seq_start = batch->q_seq_start;
  a.k_len = batch->k_len;
  a.has_layout = layout != nullptr;
  if (layout) {
    a.paged = layout->paged;
    a.k_seq_start = layout->k_seq_start;
    a.page_table = layout->page_table;
    a.page_table_stride = layout->page_table_stride;
    a.num_rows = layout->num_rows;
  }
  a.indices = indices;
  a.k = indices ? k : 0;
  a.scores = scores;
  a.ld = ld_scores;
  return hip_status(dsa::launch_validate(a, report, stream), "validate launch");
}

dsa_status_t dsa_topk(const dsa_batch_t *batch, const float *scores, int64_t ld_scores, int32_t k, int32_t *indices,
                      void *workspace, size_t workspace_bytes, hipStream_t stream) {
  dsa_status_t st = check_topk(batch, scores, ld_scores, k, indices);
  if (st != DSA_OK) return st;
  const size_t need = dsa::topk_workspace_bytes(batch->num_queries, batch->max_k_len, k);
  if (workspace_bytes < need || (need && !workspace))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "top-k needs %zu workspace bytes, got %zu", need, workspace_bytes);
  if (need && !aligned(workspace, 256)) return fail(DSA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (batch->num_queries == 0) return ok();
  return hip_status(dsa::launch_topk(to_dev(batch), batch->num_queries, batch->max_k_len, scores, ld_scores, k,
                                     indices, workspace, stream),
                    "top-k launch");
}

dsa_status_t dsa_sparse_mla_workspace_size(const dsa_batch_t *batch, dsa_dtype_t dtype, int32_t heads, int32_t d_qk,
                                           int32_t d_v, int32_t k, size_t *bytes) {
  if (!bytes) return fail(DSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  dsa_status_t st = check_batch(batch);
  if (st != DSA_OK) return st;
  if (dtype == DSA_BF16 && (d_qk != 576 || d_v != 512))
    return fail(DSA_ERR_UNSUPPORTED, "bf16 sparse MLA: d_qk must be 576 and d_v 512");
  if (k < 1 || k > 65536) return fail(DSA_ERR_INVALID_ARGUMENT, "sparse MLA: k must be in [1, 65536]");
  *bytes = mla_ws(batch, dtype, heads, d_v, k);
  return ok();
}

dsa_status_t dsa_sparse_mla_fwd(const dsa_batch_t *batch, const dsa_kv_layout_t *kv_layout, dsa_dtype_t dtype,
                                int32_t heads, int32_t d_qk, int32_t d_v, const void *q, const void *kv,
                                const int32_t *indices, int32_t k, float sm_scale, void *out, float *lse,
                                void *workspace, size_t workspace_bytes, hipStream_t stream) {
  dsa_status_t st = check_mla(batch, kv_layout, dtype, heads, d_qk, d_v, q, kv, indices, k, sm_scale, out);
  if (st != DSA_OK) return st;
  const size_t need = mla_ws(batch, dtype, heads, d_v, k);
  if (workspace_bytes < need || (need && !workspace))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "sparse MLA needs %zu workspace bytes, got %zu", need, workspace_bytes);
  if (need && !aligned(workspace, 16)) return fail(DSA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  if (batch->num_queries == 0) return ok();
  const dsa::BatchDev bt = to_dev(batch);
  const dsa::KeysDev kd = to_dev(kv_layout);
  hipError_t e;
  if (dtype == DSA_BF16)
    e = dsa::launch_mla_bf16(bt, kd, batch->num_queries, heads, q, kv, indices, k, sm_scale, out, lse, workspace,
                             stream);
  else
    e = dsa::launch_mla_f32(bt, kd, batch->num_queries, heads, d_qk, d_v, (const float *)q, (const float *)kv,
                            indices, k, sm_scale, (float *)out, lse, workspace, stream);
  return hip_status(e, "sparse MLA launch");
}

dsa_status_t dsa_forward_workspace_size(const dsa_forward_args_t *a, size_t *bytes) {
  if (!a || !bytes) return fail(DSA_ERR_INVALID_ARGUMENT, "args / bytes is NULL");
  dsa_status_t st = check_batch(&a->batch);
  if (st != DSA_OK) return st;
  if (a->top_k < 1 || a->top_k > 65536) return fail(DSA_ERR_INVALID_ARGUMENT, "top_k must be in [1, 65536]");
  *bytes = forward_ws(a).total;
  return ok();
}

dsa_status_t dsa_forward(const dsa_forward_args_t *a, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!a) return fail(DSA_ERR_INVALID_ARGUMENT, "args is NULL");
  const ForwardWs ws = forward_ws(a);
  const float *scores_chk = a->scores ? a->scores : (const float *)1;  // checked below once carved
  dsa_status_t st = check_indexer(&a->batch, &a->layout, a->index_dtype, a->h_i, a->d_i, a->q_idx, a->q_scale, a->w,
                                  a->k_idx, a->k_scale, a->index_scale, scores_chk, ws.ld);
  if (st != DSA_OK) return st;
  if (a->scores && (!aligned(a->scores, 16) || ws.ld % 4 != 0))
    return fail(DSA_ERR_INVALID_ARGUMENT, "scores must be 16-byte aligned with ld_scores % 4 == 0");
  if (a->top_k < 1 || a->top_k > 65536) return fail(DSA_ERR_INVALID_ARGUMENT, "top_k must be in [1, 65536]");
  st = check_mla(&a->batch, &a->layout, a->mla_dtype, a->heads, a->d_qk, a->d_v, a->q, a->kv, (const int32_t *)1,
                 a->top_k, a->sm_scale, a->out);
  if (st != DSA_OK) return st;
  if (workspace_bytes < ws.total || (ws.total && !workspace))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "dsa_forward needs %zu workspace bytes, got %zu", ws.total,
                workspace_bytes);
  if (ws.total && !aligned(workspace, 256)) return fail(DSA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (a->batch.num_queries == 0) return ok();
  uint8_t *base = (uint8_t *)workspace;
  float *scores = a->scores ? a->scores : (float *)(base + ws.scores_off);
  int32_t *indices = a->indices ? a->indices : (int32_t *)(base + ws.indices_off);
  void *mla_ws_ptr = base ? base + ws.mla_off : nullptr;
  const size_t mla_bytes = ws.total - ws.mla_off;

  if (ws.fused) {
    st = dsa_indexer_topk(&a->batch, &a->layout, a->index_dtype, a->h_i, a->d_i, a->q_idx, a->q_scale, a->w,
                          a->k_idx, a->k_scale, a->index_scale, a->top_k, indices, base + ws.scores_off,
                          ws.indices_off - ws.scores_off, stream);
    if (st != DSA_OK) return st;
  } else {
    st = dsa_indexer_scores(&a->batch, &a->layout, a->index_dtype, a->h_i, a->d_i, a->q_idx, a->q_scale, a->w,
                            a->k_idx, a->k_scale, a->index_scale, scores, ws.ld, stream);
    if (st != DSA_OK) return st;
    st = dsa_topk(&a->batch, scores, ws.ld, a->top_k, indices, base ? base + ws.topk_off : nullptr, ws.topk_bytes,
                  stream);
    if (st != DSA_OK) return st;
  }
  return dsa_sparse_mla_fwd(&a->batch, &a->layout, a->mla_dtype, a->heads, a->d_qk, a->d_v, a->q, a->kv, indices,
                            a->top_k, a->sm_scale, a->out, a->lse, mla_ws_ptr, mla_bytes, stream);
}

dsa_status_t dsa_indexer_topk_workspace_size(const dsa_batch_t *batch, const dsa_kv_layout_t *keys, dsa_dtype_t dtype,
                                             int32_t h_i, int32_t d_i, int32_t k, size_t *bytes) {
  if (!bytes) return fail(DSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  dsa_status_t st = check_batch(batch);
  if (st != DSA_OK) return st;
  if (!keys) return fail(DSA_ERR_INVALID_ARGUMENT, "key layout is NULL");
  if (k < 1 || k > 65536) return fail(DSA_ERR_INVALID_ARGUMENT, "k must be in [1, 65536] (got %d)", k);
  *bytes = indexer_topk_ws(batch, keys, dtype, h_i, d_i, k);
  return ok();
}

dsa_status_t dsa_indexer_topk(const dsa_batch_t *batch, const dsa_kv_layout_t *keys, dsa_dtype_t dtype, int32_t h_i,
                              int32_t d_i, const void *q_idx, const float *q_scale, const float *w, const void *k_idx,
                              const float *k_scale, float scale, int32_t k, int32_t *indices, void *workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  dsa_status_t st = check_indexer(batch, keys, dtype, h_i, d_i, q_idx, q_scale, w, k_idx, k_scale, scale,
                                  (const float *)1, batch ? batch->max_k_len : 0);
  if (st != DSA_OK) return st;
  if (k < 1 || k > 65536) return fail(DSA_ERR_INVALID_ARGUMENT, "k must be in [1, 65536] (got %d)", k);
  if (batch->num_queries > 0 && !indices) return fail(DSA_ERR_INVALID_ARGUMENT, "indices is NULL");
  const size_t need = indexer_topk_ws(batch, keys, dtype, h_i, d_i, k);
  if (workspace_bytes < need || (need && !workspace))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "indexer + top-k needs %zu workspace bytes, got %zu", need,
                workspace_bytes);
  if (need && !aligned(workspace, 256)) return fail(DSA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (batch->num_queries == 0) return ok();
  if (fused_applies(batch, keys, dtype, h_i, d_i))
    return hip_status(dsa::launch_indexer_topk_fused(to_dev(batch), to_dev(keys), batch->num_seqs,
                                                      batch->num_queries, batch->max_q_per_seq, batch->max_k_len,
                                                      h_i, (const uint8_t *)q_idx, q_scale, w, (const uint8_t *)k_idx,
                                                      k_scale, scale, k, indices, workspace, stream),
                      "fused indexer + top-k launch");
  const int64_t ld = (int64_t)round_up((size_t)batch->max_k_len, 4);
  st = dsa_indexer_scores(batch, keys, dtype, h_i, d_i, q_idx, q_scale, w, k_idx, k_scale, scale, (float *)workspace,
                          ld, stream);
  if (st != DSA_OK) return st;
  const size_t scores_bytes = round_up((size_t)batch->num_queries * ld * sizeof(float), 256);
  return dsa_topk(batch, (const float *)workspace, ld, k, indices, (char *)workspace + scores_bytes,
                  need - scores_bytes, stream);
}

dsa_status_t dsa_cache_append(const dsa_kv_layout_t *ly, int32_t num_tokens, const int32_t *seq, const int32_t *pos,
                              int32_t d_i, const float *k_new, void *k_pool, float *k_scale_pool, int32_t d_c,
                              const void *latent_new, void *latent_pool, hipStream_t stream) {
  if (!ly) return fail(DSA_ERR_INVALID_ARGUMENT, "cache append: layout is NULL");
  if (ly->paged != 0 && ly->paged != 1) return fail(DSA_ERR_INVALID_ARGUMENT, "cache append: paged must be 0 or 1");
  if (ly->num_rows < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "cache append: num_rows must be >= 1");
  if (ly->paged) {
    if (!ly->page_table) return fail(DSA_ERR_INVALID_ARGUMENT, "cache append: page_table is NULL");
    if (ly->page_size != dsa::kPageSize)
      return fail(DSA_ERR_UNSUPPORTED, "cache append: page_size %d (only %d is implemented)", ly->page_size, dsa::kPageSize);
    if (ly->page_table_stride < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "cache append: page_table_stride must be >= 1");
  } else if (!ly->k_seq_start) {
    return fail(DSA_ERR_INVALID_ARGUMENT, "cache append: k_seq_start is NULL");
  }
  if (num_tokens < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "cache append: num_tokens must be >= 0");
  if (d_i < 4 || d_i > 512 || d_i % 4 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "cache append: d_i must be a multiple of 4 in [4, 512] (got %d)", d_i);
  if (d_c < 0 || d_c > 4096 || d_c % 8 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "cache append: d_c must be 0 or a multiple of 8 up to 4096 (got %d)", d_c);
  if (num_tokens > 0) {
    if (!seq || !pos || !k_new || !k_pool || !k_scale_pool)
      return fail(DSA_ERR_INVALID_ARGUMENT, "cache append: seq, pos, k_new, k_pool and k_scale_pool must be non-NULL");
    if (!aligned(k_new, 16) || !aligned(k_pool, 4) || !aligned(k_scale_pool, 4))
      return fail(DSA_ERR_INVALID_ARGUMENT, "cache append: k_new must be 16-byte and k_pool / k_scale_pool 4-byte aligned");
    if (d_c > 0) {
      if (!latent_new || !latent_pool) return fail(DSA_ERR_INVALID_ARGUMENT, "cache append: latent_new / latent_pool is NULL");
      if (!aligned(latent_new, 16) || !aligned(latent_pool, 16))
        return fail(DSA_ERR_INVALID_ARGUMENT, "cache append: latent_new / latent_pool must be 16-byte aligned");
    }
  }
  return hip_status(dsa::launch_cache_append(to_dev(ly), num_tokens, seq, pos, d_i, k_new, k_pool, k_scale_pool, d_c,
                                             d_c > 0 ? latent_new : nullptr, d_c > 0 ? latent_pool : nullptr, stream),
                    "cache append launch");
}

}  // extern "C"
