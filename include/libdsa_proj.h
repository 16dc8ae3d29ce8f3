/* libdsa_proj: the output projections that follow the sparse stage, in a
 * library of their own (libdsa_proj.so, which links hipBLASLt and libdsa.so),
 * so that the hot-path library itself loads no GEMM library.
 *
 * Conventions are libdsa's (include/libdsa.h): device pointers, caller-owned
 * memory, asynchronous on the given stream, host-side argument checks that
 * return a dsa_status_t before anything is launched, and the failure detail
 * in libdsa's dsa_last_error().
 */
#ifndef LIBDSA_PROJ_H
#define LIBDSA_PROJ_H

#include "libdsa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------------
 * Output projections after the sparse stage ([G] Stage 2, the u_t equation;
 * the implementation section's w_uv and w_out linear layers):
 *
 *   y[t, h, :] = W_UV,h . o[t, h, :]          (d_c -> d_h, per head)
 *   out[t, :]  = W_O . concat_h y[t, h, :]      (heads * d_h -> hidden)
 *
 * Both are dense bf16 GEMMs with fp32 accumulation, run by hipBLASLt; y is
 * rounded to bf16 in the workspace between them.
 *   blaslt  a hipBLASLt handle (dsa_blaslt_create, or the caller's own
 *           hipblasLtCreate), used on `stream`
 *   o       [T, heads, d_c] bf16 (dsa_sparse_mla_fwd's output)
 *   w_uv    [heads * d_h, d_c] bf16 (rows h*d_h .. are W_UV,h)
 *   w_o     [hidden, heads * d_h] bf16
 *   out     [T, hidden] bf16
 *   d_c, d_h, hidden: multiples of 8.  workspace: 256-byte aligned,
 *   dsa_output_projection_workspace_size() bytes (y, then 32 MiB for the
 *   GEMM library).
 * ---------------------------------------------------------------------- */
dsa_status_t dsa_output_projection(void *blaslt, int32_t num_queries, int32_t heads, int32_t d_c,
                                   int32_t d_h, int32_t hidden, const void *o, const void *w_uv,
                                   const void *w_o, void *out, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream);

dsa_status_t dsa_output_projection_workspace_size(int32_t num_queries, int32_t heads, int32_t d_h,
                                                  size_t *bytes);

/* A hipBLASLt handle for dsa_output_projection (host and device resources
 * of the GEMM library; the caller owns it and destroys it). */
dsa_status_t dsa_blaslt_create(void **handle);
dsa_status_t dsa_blaslt_destroy(void *handle);

#ifdef __cplusplus
}
#endif

#endif /* LIBDSA_PROJ_H */
