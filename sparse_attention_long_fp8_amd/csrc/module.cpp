// The page's complete DSA module ("DeepSeek Sparse Attention DSA Architecture
// Guide", "End-to-End Implementation": DeepSeekSparseAttention with its
// LightningIndexer), fp32, one query token per batch element over an S-token
// history.  The page projects every history row to an indexer key and
// decompresses every selected latent row into per-head keys and values; the
// same function is computed here with each weight folded into the side that
// has one vector per batch element:
//   q_I = W_qI h_q,  q = W_Q h_q                       (gemv_rows)
//   u = W_kI^T q_I,  q_abs[h] = W_UK,h^T q[h]          (gemv_cols)
//   I[s] = ReLU(h_s . u) / sqrt(d_I)  (= ReLU(q_I . W_kI h_s) / sqrt(d_I))
//   top-k of I                                         (top-k kernel)
//   o_abs[h] = softmax_S(q_abs[h] . c_s / sqrt(d_h)) . c_s   (fp32 sparse MLA)
//   y[h] = W_UV,h o_abs[h],  out = W_out y             (gemv_rows)
#include <hip/hip_runtime.h>

#include <cmath>

#include "dsa_launch.h"
#include "libdsa.h"

namespace dsa {
dsa_status_t report(dsa_status_t st, const char *fmt, ...);  // libdsa.cpp
}  // namespace dsa

namespace {

constexpr int kModuleMaxHidden = 16384;  // the scoring kernel stages u in LDS

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct ModuleWs {
  size_t meta, q_idx, u, scores, topk, topk_bytes, q, q_abs, o_abs, y, mla, mla_bytes, total;
  int64_t ld;
};

ModuleWs module_ws(int32_t B, int32_t S, int32_t hidden, int32_t H, int32_t d_h, int32_t d_c, int32_t d_i) {
  ModuleWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += round_up(bytes, 256); return at; };
  w.ld = (int64_t)round_up((size_t)S, 4);
  w.meta = take(((size_t)B + 1) * 4 + (size_t)B * 4 + (size_t)B * 8 + (size_t)B * 4 + 64);
  w.q_idx = take((size_t)B * d_i * 4);
  w.u = take((size_t)B * hidden * 4);
  w.scores = take((size_t)B * w.ld * 4);
  w.topk_bytes = dsa::topk_workspace_bytes(B, S, S);  // the largest any top_k needs
  w.topk = take(w.topk_bytes);
  w.q = take((size_t)B * H * d_h * 4);
  w.q_abs = take((size_t)B * H * d_c * 4);
  w.o_abs = take((size_t)B * H * d_c * 4);
  w.y = take((size_t)B * H * d_h * 4);
  w.mla_bytes = dsa::mla_f32_workspace_bound(B, H, d_c);
  w.mla = take(w.mla_bytes);
  w.total = off;
  return w;
}

bool sizes_ok(int32_t batch, int32_t seq_len, int32_t hidden, int32_t heads, int32_t head_dim, int32_t latent_dim,
              int32_t index_dim) {
  return batch >= 1 && seq_len >= 1 && hidden >= 1 && heads >= 1 && head_dim >= 1 && latent_dim >= 1 &&
         index_dim >= 1;
}

bool aligned16(const void *p) { return (uintptr_t)p % 16 == 0; }

}  // namespace

extern "C" {

dsa_status_t dsa_module_forward_workspace_size(int32_t batch, int32_t seq_len, int32_t hidden, int32_t heads,
                                               int32_t head_dim, int32_t latent_dim, int32_t index_dim,
                                               size_t *bytes) {
  if (!bytes) return dsa::report(DSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (!sizes_ok(batch, seq_len, hidden, heads, head_dim, latent_dim, index_dim))
    return dsa::report(DSA_ERR_INVALID_ARGUMENT, "module forward: every size must be >= 1");
  *bytes = module_ws(batch, seq_len, hidden, heads, head_dim, latent_dim, index_dim).total;
  return dsa::report(DSA_OK, "");
}

dsa_status_t dsa_module_forward(int32_t batch, int32_t seq_len, int32_t hidden, int32_t heads, int32_t head_dim,
                                int32_t latent_dim, int32_t index_dim, int32_t top_k, const float *q_hidden,
                                const float *hist, const float *latent, const float *w_qi, const float *w_ki,
                                const float *w_q, const float *w_uk, const float *w_uv, const float *w_out,
                                float *out, int32_t *indices, void *workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  if (!sizes_ok(batch, seq_len, hidden, heads, head_dim, latent_dim, index_dim))
    return dsa::report(DSA_ERR_INVALID_ARGUMENT, "module forward: every size must be >= 1");
  if (heads > 64 || latent_dim > 256 || hidden > kModuleMaxHidden || batch > 65535)
    return dsa::report(DSA_ERR_UNSUPPORTED,
                       "module forward: needs heads <= 64, latent_dim <= 256, hidden <= %d, batch <= 65535",
                       kModuleMaxHidden);
  if (top_k < 1 || top_k > 65536) return dsa::report(DSA_ERR_INVALID_ARGUMENT, "module forward: top_k in [1, 65536]");
  if ((int64_t)batch * seq_len > INT32_MAX)
    return dsa::report(DSA_ERR_UNSUPPORTED, "module forward: batch * seq_len must fit in int32");
  if (!q_hidden || !hist || !latent || !w_qi || !w_ki || !w_q || !w_uk || !w_uv || !w_out || !out || !indices)
    return dsa::report(DSA_ERR_INVALID_ARGUMENT, "module forward: a tensor pointer is NULL");
  const ModuleWs w = module_ws(batch, seq_len, hidden, heads, head_dim, latent_dim, index_dim);
  if (workspace_bytes < w.total || !workspace)
    return dsa::report(DSA_ERR_WORKSPACE_TOO_SMALL, "module forward needs %zu workspace bytes, got %zu", w.total,
                       workspace_bytes);
  if ((uintptr_t)workspace % 256) return dsa::report(DSA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  char *base = (char *)workspace;
  const int B = batch, S = seq_len, H = heads, d_h = head_dim, d_c = latent_dim, d_i = index_dim;
  int32_t *q_seq_start = (int32_t *)(base + w.meta);
  int32_t *k_len = q_seq_start + (B + 1);
  int64_t *k_seq_start = (int64_t *)(((uintptr_t)(k_len + B) + 7) / 8 * 8);
  float *ones = (float *)(k_seq_start + B);
  float *q_idx = (float *)(base + w.q_idx), *u = (float *)(base + w.u), *scores = (float *)(base + w.scores);
  float *q = (float *)(base + w.q), *q_abs = (float *)(base + w.q_abs), *o_abs = (float *)(base + w.o_abs);
  float *y = (float *)(base + w.y);
  auto fail = [](hipError_t e, const char *what) {
    return dsa::report(DSA_ERR_HIP, "module forward, %s: %s", what, hipGetErrorString(e));
  };
  hipError_t e = dsa::launch_module_meta(B, S, q_seq_start, k_len, k_seq_start, ones, stream);
  if (e != hipSuccess) return fail(e, "batch arrays");
  // q_I = W_qI h_q and q = W_Q h_q (both rows read h_q)
  const int v_h = hidden % 4 == 0 && aligned16(q_hidden) && aligned16(w_qi) && aligned16(w_q);
  const dsa::GemvRowJob jqi{w_qi, q_hidden, q_idx, d_i, hidden, d_i, v_h, hidden, 0, d_i, 0};
  const dsa::GemvRowJob jq{w_q, q_hidden, q, H * d_h, hidden, H * d_h, v_h, hidden, 0, (int64_t)H * d_h, 0};
  if ((e = dsa::launch_gemv_rows(jqi, jq, B, stream)) != hipSuccess) return fail(e, "query projections");
  // u = W_kI^T q_I (one group) and q_abs[h] = W_UK,h^T q[h] (W_UK,h = rows h*d_h .. of w_uk)
  const dsa::GemvColJob ju{w_ki, q_idx, u, 1, d_i, hidden, d_i, 0, hidden, 0, 0};
  const dsa::GemvColJob jk{w_uk, q, q_abs, H, d_h, d_c, (int64_t)H * d_h, d_h, (int64_t)H * d_c, d_c, 0};
  if ((e = dsa::launch_gemv_cols(ju, jk, B, stream)) != hipSuccess) return fail(e, "folded queries");
  // indexer scores over each full history, then top-k
  if ((e = dsa::launch_module_scores(hist, u, B, S, hidden, 1.f / sqrtf((float)d_i), scores, w.ld, stream)) !=
      hipSuccess)
    return fail(e, "indexer scores");
  const dsa_batch_t bt{B, B, q_seq_start, k_len, 1, S};
  dsa_status_t st = dsa_topk(&bt, scores, w.ld, top_k, indices, base + w.topk, w.topk_bytes, stream);
  if (st != DSA_OK) return st;
  // softmax over the selected latent rows, per head, scale 1/sqrt(d_h)
  const dsa_kv_layout_t lat_ly{0, k_seq_start, nullptr, 0, 64, (int64_t)B * S};
  st = dsa_sparse_mla_fwd(&bt, &lat_ly, DSA_F32, H, d_c, d_c, q_abs, latent, indices, top_k,
                          1.f / sqrtf((float)d_h), o_abs, nullptr, base + w.mla, w.mla_bytes, stream);
  if (st != DSA_OK) return st;
  // y[h] = W_UV,h o_abs[h] (rows h*d_h .. of w_uv read o_abs[h]); out = W_out y
  const int v_c = d_c % 4 == 0 && aligned16(w_uv);
  const dsa::GemvRowJob juv{w_uv, o_abs, y, H * d_h, d_c, d_h, v_c, (int64_t)H * d_c, d_c, (int64_t)H * d_h, 0};
  if ((e = dsa::launch_gemv_rows(juv, dsa::GemvRowJob{}, B, stream)) != hipSuccess) return fail(e, "W_UV");
  const int v_o = (H * d_h) % 4 == 0 && aligned16(w_out);
  const dsa::GemvRowJob jo{w_out, y, out, hidden, H * d_h, hidden, v_o, (int64_t)H * d_h, 0, hidden, 0};
  if ((e = dsa::launch_gemv_rows(jo, dsa::GemvRowJob{}, B, stream)) != hipSuccess) return fail(e, "W_out");
  return dsa::report(DSA_OK, "");
}

}  // extern "C"
