// Batch arrays of the page-module entry point (one query per sequence, each
// over a full S-token history): q_seq_start[b] = b, k_len[b] = S,
// k_seq_start[b] = b*S, and the indexer's single head weight 1.  Written on
// the stream, so the entry point needs no host-to-device copy.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

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

hipError_t launch_module_meta(int batch, int seq_len, int32_t *q_seq_start, int32_t *k_len, int64_t *k_seq_start,
                              float *ones, hipStream_t stream) {
  hipLaunchKernelGGL(module_meta_kernel, dim3((batch + 1 + 255) / 256), dim3(256), 0, stream, batch, seq_len,
                     q_seq_start, k_len, k_seq_start, ones);
  return hipGetLastError();
}

}  // namespace dsa
