// Test-only probes of gfx950 instruction semantics the libdsa kernels rely
// on: FP8, bf16 and fp32 MFMA operand / accumulator lane layouts (and with them the
// FP8 E4M3 interpretation of bytes), the lane mapping of the LDS transpose
// read, and where an LDS-DMA load with an immediate offset writes.  One wave each, fully in bounds; built into libdsa_probe.so, which
// only the test-suite loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

// a, b: [64 lanes][32 bytes] operand registers as each lane holds them;
// d: [64 lanes][16] accumulator registers after one MFMA from zero.
__global__ void probe_fp8_32x32x64_kernel(const v8i *a, const v8i *b, v16f *d) {
  const int l = threadIdx.x;
  v16f acc = {};
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[l], b[l], acc, 0, 0, 0, 127, 0, 127);
  d[l] = acc;
}

// a, b: [64][8] bf16; d: [64][4]
__global__ void probe_bf16_16x16x32_kernel(const v8bf *a, const v8bf *b, v4f *d) {
  const int l = threadIdx.x;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[l], b[l], acc, 0, 0, 0);
  d[l] = acc;
}

// a, b: [64][8] bf16; d: [64][16]
__global__ void probe_bf16_32x32x16_kernel(const v8bf *a, const v8bf *b, v16f *d) {
  const int l = threadIdx.x;
  v16f acc = {};
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[l], b[l], acc, 0, 0, 0);
  d[l] = acc;
}

// a, b: [64] fp32; d: [64][4]
__global__ void probe_f32_16x16x4_kernel(const float *a, const float *b, v4f *d) {
  const int l = threadIdx.x;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[l], b[l], acc, 0, 0, 0);
  d[l] = acc;
}

// src: 4096 16-bit words copied into LDS; off: per-lane byte offset (8-byte
// aligned, < 8192 - 8, checked on the host); dst: [64][4] words read back.
__global__ void probe_tr16_kernel(const short *src, const int *off, v4s *dst) {
  __shared__ short lds[4096];
  for (int i = threadIdx.x; i < 4096; i += 64) lds[i] = src[i];
  __syncthreads();
  const int o = off[threadIdx.x];
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  dst[threadIdx.x] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)((char *)lds + o));
}

// One wave's 16-byte global -> LDS load (global_load_lds_dwordx4) with a
// 256-byte immediate offset in the instruction and M0 = the LDS buffer's base.
// src holds 2048 bytes (lane l reads src + 16 l + 256, inside them); the 4 KB
// LDS buffer is zeroed before the load and copied to dst (4096 bytes) after
// it, so that the caller sees where the wave's 1 KB landed: at 16 l, or at
// 16 l + 256 if the immediate offsets the LDS address too.  Either way every
// byte written lies inside the buffer.
__global__ void probe_dma_offset_kernel(const uint8_t *src, int4 *dst) {
  __shared__ int4 lds[256];
  for (int i = threadIdx.x; i < 256; i += 64) lds[i] = int4{0, 0, 0, 0};
  __syncthreads();
  const uint32_t base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds);
  const uint8_t *g = src + 16 * threadIdx.x;
  uint32_t saved;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off offset:256\n\t"
      "s_waitcnt vmcnt(0)\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(g)
      : "memory");
  __syncthreads();
  for (int i = threadIdx.x; i < 256; i += 64) dst[i] = lds[i];
}

// Plain 16-byte-per-lane copy: the known-size reference that HBM traffic
// counters of the other kernels are scaled by.
__global__ void copy_kernel(const int4 *src, int4 *dst, long long n16) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n16;
       i += (long long)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

extern "C" {

int dsa_probe_copy(const void *src, void *dst, long long bytes, hipStream_t stream) {
  if (bytes % 16) return -1;
  hipLaunchKernelGGL(copy_kernel, dim3(4096), dim3(256), 0, stream, (const int4 *)src, (int4 *)dst,
                     bytes / 16);
  return (int)hipGetLastError();
}

int dsa_probe_fp8_32x32x64(const void *a, const void *b, float *d, hipStream_t stream) {
  hipLaunchKernelGGL(probe_fp8_32x32x64_kernel, dim3(1), dim3(64), 0, stream, (const v8i *)a,
                     (const v8i *)b, (v16f *)d);
  return (int)hipGetLastError();
}

int dsa_probe_bf16_16x16x32(const void *a, const void *b, float *d, hipStream_t stream) {
  hipLaunchKernelGGL(probe_bf16_16x16x32_kernel, dim3(1), dim3(64), 0, stream, (const v8bf *)a,
                     (const v8bf *)b, (v4f *)d);
  return (int)hipGetLastError();
}

int dsa_probe_bf16_32x32x16(const void *a, const void *b, float *d, hipStream_t stream) {
  hipLaunchKernelGGL(probe_bf16_32x32x16_kernel, dim3(1), dim3(64), 0, stream, (const v8bf *)a,
                     (const v8bf *)b, (v16f *)d);
  return (int)hipGetLastError();
}

int dsa_probe_f32_16x16x4(const void *a, const void *b, float *d, hipStream_t stream) {
  hipLaunchKernelGGL(probe_f32_16x16x4_kernel, dim3(1), dim3(64), 0, stream, (const float *)a,
                     (const float *)b, (v4f *)d);
  return (int)hipGetLastError();
}

int dsa_probe_tr16(const void *src, const int *off_host, const int *off_dev, void *dst,
                   hipStream_t stream) {
  for (int i = 0; i < 64; ++i)
    if (off_host[i] < 0 || off_host[i] > 8192 - 8 || (off_host[i] & 7)) return -1;
  hipLaunchKernelGGL(probe_tr16_kernel, dim3(1), dim3(64), 0, stream, (const short *)src, off_dev,
                     (v4s *)dst);
  return (int)hipGetLastError();
}

// src: 2048 bytes, dst: 4096 bytes (device); see probe_dma_offset_kernel.
int dsa_probe_dma_offset(const void *src, void *dst, hipStream_t stream) {
  hipLaunchKernelGGL(probe_dma_offset_kernel, dim3(1), dim3(64), 0, stream, (const uint8_t *)src, (int4 *)dst);
  return (int)hipGetLastError();
}

}  // extern "C"
