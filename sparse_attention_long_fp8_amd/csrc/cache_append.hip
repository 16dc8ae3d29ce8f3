// Decode-step cache append (gfx950).
//
// Before a decoding step scores its history, each new token's entries must be
// in the caches that step reads: its indexer key in FP8 with one fp32 scale
// per token ("DeepSeek Sparse Attention DSA Architecture Guide", "Stage 1:
// The Lightning Indexer", item 1), and its latent row, the cached c^KV that
// the sparse stage gathers ("Stage 2: Fine-Grained Token Selection").  "Sparse
// Attention Architectures for Long-Context Inference: Evolution and
// Engineering Practices", section 6, names this per-step cache update; the
// pools may be paged ("Sparse Attention in Large Language Models: Architecture
// Evolution and Engineering Practice", section 4.1).
//
// One wave per token.  The key's amax is a wave reduction; scale = amax / 448
// (1 for an all-zero row) and each code is the hardware round-to-nearest-even
// conversion of x / scale clamped to +-448, four codes packed per 4-byte
// store.  The latent row is copied in 16-byte pieces.  The rows touched are
// exactly the addressed ones.
#include <hip/hip_bf16.h>

#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kAppendWaves = 4;  // tokens per workgroup
constexpr float kE4M3Max = 448.f;

__global__ __launch_bounds__(kAppendWaves * 64) void cache_append_kernel(
    KeysDev kd, int num_tokens, const int32_t *__restrict__ seq, const int32_t *__restrict__ pos,
    int d_i, const float *__restrict__ k_new, uint8_t *__restrict__ k_pool,
    float *__restrict__ k_scale_pool, int d_c, const uint16_t *__restrict__ lat_new,
    uint16_t *__restrict__ lat_pool) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * kAppendWaves + (int)(threadIdx.x >> 6);
  if (i >= num_tokens) return;
  const int64_t row = key_row(kd, seq[i], pos[i]);

  // key: lane holds elements 4c .. 4c+3 for chunks c = lane + 64u (d_i <= 512)
  const int nc = d_i >> 2;
  const float *x = k_new + (int64_t)i * d_i;
  float4 v[2];
  float amax = 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = lane + 64 * u;
    v[u] = c < nc ? *(const float4 *)(x + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
  }
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float sc = amax > 0.f ? amax / kE4M3Max : 1.f;
  auto code = [&](float f) { return fminf(fmaxf(f / sc, -kE4M3Max), kE4M3Max); };
  uint8_t *dst = k_pool + row * d_i;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = lane + 64 * u;
    if (c < nc) {
      int packed = __builtin_amdgcn_cvt_pk_fp8_f32(code(v[u].x), code(v[u].y), 0, false);
      packed = __builtin_amdgcn_cvt_pk_fp8_f32(code(v[u].z), code(v[u].w), packed, true);
      *(int *)(dst + 4 * c) = packed;
    }
  }
  if (lane == 0) k_scale_pool[row] = sc;

  // latent row: 8 bf16 per 16-byte piece
  if (d_c > 0) {
    const uint16_t *src = lat_new + (int64_t)i * d_c;
    uint16_t *out = lat_pool + row * d_c;
    for (int c = lane; c < (d_c >> 3); c += 64) *(int4 *)(out + 8 * c) = *(const int4 *)(src + 8 * c);
  }
}

hipError_t launch_cache_append(const KeysDev &kd, int num_tokens, const int32_t *seq,
                               const int32_t *pos, int d_i, const float *k_new, void *k_pool,
                               float *k_scale_pool, int d_c, const void *latent_new,
                               void *latent_pool, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const dim3 grid((num_tokens + kAppendWaves - 1) / kAppendWaves);
  hipLaunchKernelGGL(cache_append_kernel, grid, dim3(kAppendWaves * 64), 0, stream, kd, num_tokens, seq,
                     pos, d_i, k_new, (uint8_t *)k_pool, k_scale_pool, d_c,
                     (const uint16_t *)latent_new, (uint16_t *)latent_pool);
  return hipGetLastError();
}

}  // namespace dsa
