// Kernels of the page-module entry point ("DeepSeek Sparse Attention DSA
// Architecture Guide", "End-to-End Implementation": DeepSeekSparseAttention
// with its LightningIndexer), fp32, one query token per batch element.
//
// Every projection of that module multiplies a weight matrix by one vector
// per batch element, so they are matrix-vector products bound by reading
// the weights once:
//   * gemv_rows_kernel: y[b, r] = W[r, :] . x[b, group(r), :]   (one wave per
//     output row, every batch element at once);
//   * gemv_cols_kernel: y[b, g, c] = sum_j W[g*J + j, c] x[b, g, j]  (the
//     transposed product: 64 columns per workgroup, the J rows split over
//     its four waves and summed through LDS);
//   * module_scores_kernel: the indexer scores with W_kI folded into the
//     query, I[b, s] = ReLU(h_s . u_b) / sqrt(d_I), u_b = W_kI^T q_I[b]
//     (the same value as ReLU(q_I . (W_kI h_s)) / sqrt(d_I): one stream over
//     the history instead of an S x d_I key projection).
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kGemvB = 4;  // batch elements per pass over a weight row

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__global__ void module_meta_kernel(int batch, int seq_len, int32_t *q_seq_start, int32_t *k_len,
                                   int64_t *k_seq_start, float *ones) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b <= batch) q_seq_start[b] = b;
  if (b < batch) {
    k_len[b] = seq_len;
    k_seq_start[b] = (int64_t)b * seq_len;
    ones[b] = 1.f;
  }
}

__device__ void gemv_rows(const GemvRowJob &j, int blk, int batch) {
  const int lane = threadIdx.x & 63;
  const int r = blk * 4 + (threadIdx.x >> 6);
  if (r >= j.rows) return;
  const float *wr = j.w + (int64_t)r * j.cols;
  const float *xr = j.x + (int64_t)(r / j.rows_per_group) * j.x_g_stride;
  for (int b0 = 0; b0 < batch; b0 += kGemvB) {
    float acc[kGemvB] = {0.f, 0.f, 0.f, 0.f};
    if (j.vec4) {
#pragma unroll 4
      for (int c = 4 * lane; c < j.cols; c += 256) {
        const float4 wv = *(const float4 *)(wr + c);
#pragma unroll
        for (int bb = 0; bb < kGemvB; ++bb) {
          if (b0 + bb < batch) {
            const float4 xv = *(const float4 *)(xr + (int64_t)(b0 + bb) * j.x_b_stride + c);
            acc[bb] = fmaf(wv.x, xv.x, fmaf(wv.y, xv.y, fmaf(wv.z, xv.z, fmaf(wv.w, xv.w, acc[bb]))));
          }
        }
      }
    } else {
#pragma unroll 4
      for (int c = lane; c < j.cols; c += 64) {
        const float wv = wr[c];
#pragma unroll
        for (int bb = 0; bb < kGemvB; ++bb)
          if (b0 + bb < batch) acc[bb] = fmaf(wv, xr[(int64_t)(b0 + bb) * j.x_b_stride + c], acc[bb]);
      }
    }
#pragma unroll
    for (int bb = 0; bb < kGemvB; ++bb) {
      const float s = wave_sum_f(acc[bb]);
      if (lane == 0 && b0 + bb < batch) j.y[(int64_t)(b0 + bb) * j.y_b_stride + r] = s;
    }
  }
}

__global__ __launch_bounds__(256) void gemv_rows_kernel(GemvRowJob j0, GemvRowJob j1, int batch) {
  const int blk = blockIdx.x;
  if (blk < j0.blocks)
    gemv_rows(j0, blk, batch);
  else
    gemv_rows(j1, blk - j0.blocks, batch);
}

struct GemvColsLds {
  float part[4][kGemvB][64];
};

__device__ void gemv_cols(const GemvColJob &j, int blk, int batch, GemvColsLds &sh) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int cb = (j.cols + 63) / 64;
  const int g = blk / cb;
  const int c = (blk - g * cb) * 64 + lane;
  const float *wg = j.w + (int64_t)g * j.J * j.cols;
  const float *xg = j.x + (int64_t)g * j.x_g_stride;
  for (int b0 = 0; b0 < batch; b0 += kGemvB) {
    float acc[kGemvB] = {0.f, 0.f, 0.f, 0.f};
    if (c < j.cols) {
#pragma unroll 16
      for (int jj = wave; jj < j.J; jj += 4) {
        const float wv = wg[(int64_t)jj * j.cols + c];
#pragma unroll
        for (int bb = 0; bb < kGemvB; ++bb)
          if (b0 + bb < batch) acc[bb] = fmaf(wv, xg[(int64_t)(b0 + bb) * j.x_b_stride + jj], acc[bb]);
      }
    }
#pragma unroll
    for (int bb = 0; bb < kGemvB; ++bb) sh.part[wave][bb][lane] = acc[bb];
    __syncthreads();
    if (wave == 0 && c < j.cols) {
#pragma unroll
      for (int bb = 0; bb < kGemvB; ++bb)
        if (b0 + bb < batch)
          j.y[(int64_t)(b0 + bb) * j.y_b_stride + (int64_t)g * j.y_g_stride + c] =
              (sh.part[0][bb][lane] + sh.part[1][bb][lane]) + (sh.part[2][bb][lane] + sh.part[3][bb][lane]);
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void gemv_cols_kernel(GemvColJob j0, GemvColJob j1, int batch) {
  __shared__ GemvColsLds sh;
  const int blk = blockIdx.x;
  if (blk < j0.blocks)
    gemv_cols(j0, blk, batch, sh);
  else
    gemv_cols(j1, blk - j0.blocks, batch, sh);
}

// scores[b, s] = max(hist[b, s, :] . u[b, :], 0) * scale for s < S; a
// workgroup takes 16 rows of one batch element, each wave 4 of them with
// all their loads in flight (16 float4 per lane at hidden = 1024), and many
// workgroups share a CU.  u[b] sits in LDS.
constexpr int kScoreRows = 16;

__global__ __launch_bounds__(256) void module_scores_kernel(const float *__restrict__ hist,
                                                            const float *__restrict__ u, int S, int hidden,
                                                            float scale, float *__restrict__ scores, int64_t ld,
                                                            int vec4) {
  extern __shared__ float u_s[];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const float *ub = u + (int64_t)b * hidden;
  for (int c = threadIdx.x; c < hidden; c += 256) u_s[c] = ub[c];
  __syncthreads();
  const int row_end = min(S, (blockIdx.x + 1) * kScoreRows);
  const float *hb = hist + (int64_t)b * S * hidden;
  for (int r0 = blockIdx.x * kScoreRows + 4 * wave; r0 < row_end; r0 += 16) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (vec4) {
#pragma unroll 4
      for (int c = 4 * lane; c < hidden; c += 256) {
        const float4 uv = *(const float4 *)&u_s[c];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (r0 + i < row_end) {
            const float4 hv = *(const float4 *)(hb + (int64_t)(r0 + i) * hidden + c);
            acc[i] = fmaf(hv.x, uv.x, fmaf(hv.y, uv.y, fmaf(hv.z, uv.z, fmaf(hv.w, uv.w, acc[i]))));
          }
        }
      }
    } else {
#pragma unroll 4
      for (int c = lane; c < hidden; c += 64) {
        const float uv = u_s[c];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (r0 + i < row_end) acc[i] = fmaf(hb[(int64_t)(r0 + i) * hidden + c], uv, acc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s = wave_sum_f(acc[i]);
      if (lane == i && r0 + i < row_end) scores[(int64_t)b * ld + r0 + i] = fmaxf(s, 0.f) * scale;
    }
  }
}

hipError_t launch_module_meta(int batch, int seq_len, int32_t *q_seq_start, int32_t *k_len, int64_t *k_seq_start,
                              float *ones, hipStream_t stream) {
  hipLaunchKernelGGL(module_meta_kernel, dim3((batch + 1 + 255) / 256), dim3(256), 0, stream, batch, seq_len,
                     q_seq_start, k_len, k_seq_start, ones);
  return hipGetLastError();
}

hipError_t launch_gemv_rows(GemvRowJob j0, GemvRowJob j1, int batch, hipStream_t stream) {
  j0.blocks = (j0.rows + 3) / 4;
  j1.blocks = j1.w ? (j1.rows + 3) / 4 : 0;
  hipLaunchKernelGGL(gemv_rows_kernel, dim3(j0.blocks + j1.blocks), dim3(256), 0, stream, j0, j1, batch);
  return hipGetLastError();
}

hipError_t launch_gemv_cols(GemvColJob j0, GemvColJob j1, int batch, hipStream_t stream) {
  j0.blocks = (j0.cols + 63) / 64 * j0.groups;
  j1.blocks = j1.w ? (j1.cols + 63) / 64 * j1.groups : 0;
  hipLaunchKernelGGL(gemv_cols_kernel, dim3(j0.blocks + j1.blocks), dim3(256), 0, stream, j0, j1, batch);
  return hipGetLastError();
}

hipError_t launch_module_scores(const float *hist, const float *u, int batch, int S, int hidden, float scale,
                                float *scores, int64_t ld, hipStream_t stream) {
  const int vec4 = hidden % 4 == 0 && (uintptr_t)hist % 16 == 0 && (uintptr_t)u % 16 == 0;
  hipLaunchKernelGGL(module_scores_kernel, dim3((S + kScoreRows - 1) / kScoreRows, batch), dim3(256),
                     (size_t)hidden * sizeof(float), stream, hist, u, S, hidden, scale, scores, ld, vec4);
  return hipGetLastError();
}

}  // namespace dsa
