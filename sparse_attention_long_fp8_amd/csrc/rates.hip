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

}  // namespace

extern "C" {

// kind 0-2: MFMA rate probes (see rate_kernel) with `valu` in {0, 16, 32}
// VALU FMAs per MFMA (kind 2) or 0 (kinds 0, 1); kind 3: VALU only, 64 FMAs
// per iteration; kind 4: LDS reads (threads = 256, 512 or 1024 per block).
// blocks <= 4096; out holds blocks x 1024 floats.  Returns 0, or -1 for an
// unsupported combination (nothing launched).
int dsa_probe_rate(int kind, int valu, int blocks, int threads, int iters, float *out, hipStream_t stream) {
  if (blocks < 1 || blocks > 4096 || iters < 1) return -1;
  const dim3 g(blocks), b(256);
  if (kind == 4) {
    if (threads != 256 && threads != 512 && threads != 1024) return -1;
    hipLaunchKernelGGL(lds_rate_kernel, g, dim3(threads), 0, stream, out, iters);
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
