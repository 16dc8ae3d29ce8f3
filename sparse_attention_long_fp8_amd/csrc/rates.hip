// Test-only throughput probes of gfx950: dense MFMA rates with independent
// accumulators, the wave64 VALU issue rate, VALU work beside running MFMAs,
// and conflict-free LDS read bandwidth.  They give the realistic ceilings the
// kernels' rooflines are read against.  Every kernel loops over registers (and,
// for the LDS probe, a 64 KB LDS buffer with masked indices): no global access
// but one store per thread of a result into `out` (blocks x 256 floats; the
// LDS probe takes blockDim <= 1024, so blocks x 1024).  Built into
// libdsa_probe.so, which only the test-suite loads.
#include <hip/hip_runtime.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// eight independent fp32 FMAs (x[i] += m1 * m2), written out so that the
// compiler can neither merge nor drop them
#define DSA_FMA8(x)                                                          \
  asm volatile("v_fmac_f32 %0, %8, %9\n v_fmac_f32 %1, %8, %9\n"             \
               "v_fmac_f32 %2, %8, %9\n v_fmac_f32 %3, %8, %9\n"             \
               "v_fmac_f32 %4, %8, %9\n v_fmac_f32 %5, %8, %9\n"             \
               "v_fmac_f32 %6, %8, %9\n v_fmac_f32 %7, %8, %9"               \
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), \
                 "+v"(x[5]), "+v"(x[6]), "+v"(x[7])                          \
               : "v"(m1), "v"(m2))

// KIND 0: bf16 16x16x32, four accumulators; 1: bf16 32x32x16, two;
// 2: FP8 32x32x64 (scaled form, unit scales), two.  NM MFMAs and 8*NV8 VALU
// FMAs per iteration.
template <int KIND, int NM, int NV8>
__global__ __launch_bounds__(256) void rate_kernel(float *out, int iters, int seed) {
  const int tid = threadIdx.x;
  v8bf ab, bb;
  v8i a8, b8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ab[i] = (__bf16)(float)(seed + i);
    bb[i] = (__bf16)(float)(tid + i);
    a8[i] = seed * 0x01010101 + i;
    b8[i] = tid + i;
  }
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = tid * 0.001f + i;
  const float m1 = 0.999f, m2 = 0.001f * seed;
  v4f c0{}, c1{}, c2{}, c3{};
  v16f d0{}, d1{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if constexpr (KIND == 0) {
        switch (m & 3) {
          case 0: c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, bb, c0, 0, 0, 0); break;
          case 1: c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, bb, c1, 0, 0, 0); break;
          case 2: c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, bb, c2, 0, 0, 0); break;
          default: c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, bb, c3, 0, 0, 0); break;
        }
      } else if constexpr (KIND == 1) {
        if (m & 1) d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, d1, 0, 0, 0);
        else d0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, d0, 0, 0, 0);
      } else {
        if (m & 1) d1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, d1, 0, 0, 0, 127, 0, 127);
        else d0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, d0, 0, 0, 0, 127, 0, 127);
      }
    }
#pragma unroll
    for (int v = 0; v < NV8; ++v) DSA_FMA8(x);
  }
  float s = c0[0] + c1[1] + c2[2] + c3[3] + d0[0] + d1[5];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * 256 + tid] = s;
}

// Eight conflict-free 16-byte LDS reads per thread and iteration: a wave reads
// 1 KB of consecutive bytes per instruction.
__global__ __launch_bounds__(1024) void lds_rate_kernel(float *out, int iters) {
  __shared__ v4i buf[4096];  // 64 KB
  for (int i = threadIdx.x; i < 4096; i += blockDim.x) buf[i] = v4i{i, i + 1, i + 2, i + 3};
  __syncthreads();
  v4i acc = v4i{0, 0, 0, 0};
  const int base = (threadIdx.x & 63) + 64 * ((threadIdx.x >> 6) & 7);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) acc += buf[(base + 512 * r + it) & 4095];
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc.x + acc.y + acc.z + acc.w);
}

// LDS reads in the access patterns of the attention kernel's tile (rows of
// 1040 bytes; 32 tokens), eight per thread and iteration, every address inside
// the 64 KB buffer:
//   P = 0: 16-byte reads, lane l at byte 16 l of a 1 KB block (the plain case);
//   P = 1: 16-byte QK operand reads: lane (g = l / 16, m = l % 16) reads token
//          tok(m) of a 16-token half at byte 16 g + 64 ks (ks = 0 .. 15);
//   P = 2: the same with token m (no permutation);
//   P = 3: 8-byte reads, lane l at byte 8 l of a 512-byte block (plain);
//   P = 4: 8-byte transpose reads of the P.V product: lane (g, n) reads token
//          tok(4 g + n / 4) at byte 8 (n % 4) + 32 nt (nt = 0 .. 31).
__device__ __forceinline__ int probe_tok(int m) { return 4 * (m & 3) + (((m >> 1) & 2) | ((m >> 3) & 1)); }

template <int P>
__global__ __launch_bounds__(1024) void lds_pattern_kernel(float *out, int iters) {
  __shared__ v4i buf[4096];  // 64 KB
  for (int i = threadIdx.x; i < 4096; i += blockDim.x) buf[i] = v4i{i, i + 1, i + 2, i + 3};
  __syncthreads();
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int wave = threadIdx.x >> 6;
  const uint8_t *base = (const uint8_t *)buf + (wave & 1) * 32768;  // two tiles' worth
  int off;
  if constexpr (P == 0) off = 16 * lane;
  else if constexpr (P == 1) off = probe_tok(n) * 1040 + 16 * g;
  else if constexpr (P == 2) off = n * 1040 + 16 * g;
  else if constexpr (P == 3) off = 8 * lane;
  else off = probe_tok(4 * g + (n >> 2)) * 1040 + 8 * (n & 3);
  // the second iteration's reads sit `step` bytes further; the offset is made
  // opaque in every iteration so that the loads are not hoisted out of the loop
  constexpr int step = P == 0 ? 8192 : P == 4 ? 128 : 256;
  v4i acc = v4i{0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
    int o = off + (it & 1) * step;
    __asm__ volatile("" : "+v"(o));
    const uint8_t *b = base + o;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if constexpr (P == 0) {
        acc += *(const v4i *)(b + 1024 * r);
      } else if constexpr (P == 1 || P == 2) {
        acc += *(const v4i *)(b + 16 * 1040 * (r & 1) + 64 * (r >> 1));
      } else if constexpr (P == 3) {
        const int2 v = *(const int2 *)(b + 4096 * r);  // (the compiler pairs them: ds_read2st64_b64)
        acc.x += v.x;
        acc.y += v.y;
      } else {
        const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(b + 16 * 1040 * (r & 1) + 32 * (r >> 1)));
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc.x + acc.y + acc.z + acc.w);
}

// LDS reads at per-lane offsets from a table: read r (0..7) of lane l is at
// byte tab[64 r + l] of a 32 KB half of the buffer (waves alternate halves),
// plus `step` bytes in odd iterations.  W = 16: 16-byte reads; W = 8: 8-byte
// transpose reads (ds_read_tr16_b64).  The host keeps every offset + step + W
// within 32 KB and aligned to W.
template <int W>
__global__ __launch_bounds__(1024) void lds_table_kernel(float *out, const int *__restrict__ tab, int iters, int step) {
  __shared__ v4i buf[4096];  // 64 KB
  for (int i = threadIdx.x; i < 4096; i += blockDim.x) buf[i] = v4i{i, i + 1, i + 2, i + 3};
  const int lane = threadIdx.x & 63;
  int offs[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) offs[r] = tab[64 * r + lane];
  __syncthreads();
  const uint8_t *base = (const uint8_t *)buf + ((threadIdx.x >> 6) & 1) * 32768;
  v4i acc = v4i{0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
    int o = (it & 1) * step;
    __asm__ volatile("" : "+v"(o));
    const uint8_t *b = base + o;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if constexpr (W == 16) {
        acc += *(const v4i *)(b + offs[r]);
      } else {
        const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(b + offs[r]));
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc.x + acc.y + acc.z + acc.w);
}

}  // namespace

extern "C" {

// LDS reads at the offsets of `tab` (512 ints on the device, see
// lds_table_kernel): width 16 or 8 (transpose reads); threads 256, 512 or
// 1024; blocks <= 4096; out holds blocks x threads floats.  The caller keeps
// every offset + step + width within 32768 and aligned to the width.  Returns
// 0, or -1 for an unsupported combination (nothing launched).
int dsa_probe_lds_table(int width, const int *tab, int step, int blocks, int threads, int iters, float *out,
                        hipStream_t stream) {
  if (blocks < 1 || blocks > 4096 || iters < 1 || step < 0 || (threads != 256 && threads != 512 && threads != 1024))
    return -1;
  if (width == 16) hipLaunchKernelGGL(lds_table_kernel<16>, dim3(blocks), dim3(threads), 0, stream, out, tab, iters, step);
  else if (width == 8) hipLaunchKernelGGL(lds_table_kernel<8>, dim3(blocks), dim3(threads), 0, stream, out, tab, iters, step);
  else return -1;
  return (int)hipGetLastError();
}

// kind 0-2: MFMA rate probes (see rate_kernel) with `valu` in {0, 16, 32}
// VALU FMAs per MFMA (kind 2) or 0 (kinds 0, 1); kind 3: VALU only, 64 FMAs
// per iteration; kind 4: LDS reads (threads = 256, 512 or 1024 per block);
// kinds 5-9: LDS reads in pattern 0-4 of lds_pattern_kernel (same threads).
// blocks <= 4096; out holds blocks x 1024 floats.  Returns 0, or -1 for an
// unsupported combination (nothing launched).
int dsa_probe_rate(int kind, int valu, int blocks, int threads, int iters, float *out, hipStream_t stream) {
  if (blocks < 1 || blocks > 4096 || iters < 1) return -1;
  const dim3 g(blocks), b(256);
  if (kind >= 4 && kind <= 9) {
    if (threads != 256 && threads != 512 && threads != 1024) return -1;
    const dim3 b(threads);
    switch (kind) {
      case 4: hipLaunchKernelGGL(lds_rate_kernel, g, b, 0, stream, out, iters); break;
      case 5: hipLaunchKernelGGL(lds_pattern_kernel<0>, g, b, 0, stream, out, iters); break;
      case 6: hipLaunchKernelGGL(lds_pattern_kernel<1>, g, b, 0, stream, out, iters); break;
      case 7: hipLaunchKernelGGL(lds_pattern_kernel<2>, g, b, 0, stream, out, iters); break;
      case 8: hipLaunchKernelGGL(lds_pattern_kernel<3>, g, b, 0, stream, out, iters); break;
      default: hipLaunchKernelGGL(lds_pattern_kernel<4>, g, b, 0, stream, out, iters); break;
    }
    return (int)hipGetLastError();
  }
  if (threads != 256) return -1;
  if (kind == 0 && valu == 0) hipLaunchKernelGGL((rate_kernel<0, 4, 0>), g, b, 0, stream, out, iters, 1);
  else if (kind == 1 && valu == 0) hipLaunchKernelGGL((rate_kernel<1, 2, 0>), g, b, 0, stream, out, iters, 1);
  else if (kind == 2 && valu == 0) hipLaunchKernelGGL((rate_kernel<2, 2, 0>), g, b, 0, stream, out, iters, 1);
  else if (kind == 2 && valu == 16) hipLaunchKernelGGL((rate_kernel<2, 2, 4>), g, b, 0, stream, out, iters, 1);
  else if (kind == 2 && valu == 32) hipLaunchKernelGGL((rate_kernel<2, 2, 8>), g, b, 0, stream, out, iters, 1);
  else if (kind == 3) hipLaunchKernelGGL((rate_kernel<2, 0, 8>), g, b, 0, stream, out, iters, 1);
  else return -1;
  return (int)hipGetLastError();
}

}  // extern "C"
