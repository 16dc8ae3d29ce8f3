// Device-side helpers shared by the libdsa kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

// Batch description as the kernels see it (device arrays).
struct BatchDev {
  int32_t num_seqs;
  const int32_t *q_seq_start;  // [B+1]
  const int32_t *k_len;        // [B]
  // every sequence has exactly one query row (q_seq_start[b] == b, the
  // decode batch): row t is sequence t, and its candidates are k_len[t]
  int32_t one_per_seq;
};

// Key addressing: contiguous rows or 64-token pages.
struct KeysDev {
  int32_t paged;
  const int64_t *k_seq_start;  // [B] (contiguous)
  const int32_t *page_table;   // [B, stride] (paged)
  int32_t stride;
};

constexpr int kPageShift = 6;  // 64-token pages
constexpr int kPageSize = 1 << kPageShift;

// Sequence that owns query row t: the largest b with q_seq_start[b] <= t.
__device__ __forceinline__ int seq_of_row(const BatchDev &bt, int t) {
  if (bt.one_per_seq) return t;
  int lo = 0, hi = bt.num_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (bt.q_seq_start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The same sequence, found by a whole wave (every lane active) in a 64-ary
// search: lane l reads entry b + l * step and a ballot of the entries <= t
// picks the bracket, so up to 64 sequences cost one memory round trip (a
// binary search pays one per halving).  Entries are non-decreasing; the
// result is wave-uniform and in [0, num_seqs) for any array contents.
__device__ __forceinline__ int seq_of_row_wave(const BatchDev &bt, int t) {
  if (bt.one_per_seq) return t;
  const int lane = __lane_id();
  int b = 0;
  for (int span = bt.num_seqs; span > 1;) {
    const int step = (span + 63) >> 6;
    const int pos = b + lane * step;
    const bool le = pos < b + span && bt.q_seq_start[pos] <= t;
    const int c = max((int)__popcll(__ballot(le)), 1);
    b += (c - 1) * step;
    span = min(step, span - (c - 1) * step);
  }
  return __builtin_amdgcn_readfirstlane(b);
}

// Query row t of sequence b sits at p = k_len[b] - nq_b + (t - q_seq_start[b])
// and has n = p + 1 causal candidates (itself included).
__device__ __forceinline__ int candidates_of_row(const BatchDev &bt, int b, int t) {
  if (bt.one_per_seq) return bt.k_len[b];
  int q0 = bt.q_seq_start[b];
  int nq = bt.q_seq_start[b + 1] - q0;
  return bt.k_len[b] - nq + (t - q0) + 1;
}

// Flat row (contiguous row, or page * 64 + slot of the pool) of key s of sequence b.
__device__ __forceinline__ int64_t key_row(const KeysDev &kd, int b, int s) {
  if (!kd.paged) return kd.k_seq_start[b] + s;
  int page = kd.page_table[(int64_t)b * kd.stride + (s >> kPageShift)];
  return ((int64_t)page << kPageShift) + (s & (kPageSize - 1));
}

// Order-preserving map float -> uint32 (a > b  <=>  key(a) > key(b));
// -0 is folded onto +0 so that they compare equal.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The score of an order-preserving key (inverse of float_key; +0 for the key
// of +0 and -0).
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// The lane index, computed where it is used: the compiler can neither hoist
// nor share it, so no register holds it across a loop.
__device__ __forceinline__ int opaque_lane_id() {
  int l;
  __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

typedef __attribute__((address_space(3))) void lds_ptr_t;

// 16-byte global -> LDS load for a whole wave: lane i's 16 bytes land at LDS
// byte address lds_byte + 16 * i (lds_byte must be wave-uniform).  Written as
// inline assembly so that the compiler does not treat every later LDS read as
// possibly aliasing it (it would otherwise drain all such loads before them);
// callers wait for completion with an explicit vmcnt wait.  M0, which carries
// the LDS base, is saved and restored inside the block.
__device__ __forceinline__ void lds_dma16_at(const void *gaddr, uint32_t lds_byte) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_byte);
  uint32_t saved;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(gaddr)
      : "memory");
}

// The same load from gaddr + OFF, OFF an immediate byte offset in the
// instruction (0 <= OFF < 4096), so that loads from one per-lane base need no
// address arithmetic of their own.  The instruction adds OFF to the LDS
// address as well (pinned by a probe), so M0 is set to lds_byte - OFF: lane
// i's 16 bytes still land at lds_byte + 16 * i.  Needs lds_byte >= OFF.
template <int OFF>
__device__ __forceinline__ void lds_dma16_imm(const void *gaddr, uint32_t lds_byte) {
  static_assert(OFF >= 0 && OFF < 4096, "immediate offset range");
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_byte) - (uint32_t)OFF;
  uint32_t saved;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off offset:%3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(gaddr), "n"(OFF)
      : "memory");
}

// The same 16-byte load from one wave-uniform base address: lane i's 16
// bytes come from sbase + voff (voff a per-lane byte offset) and land at LDS
// byte address lds_byte + 16 * i.  The base is held in scalar registers, so
// the lanes' addresses cost no vector arithmetic.
__device__ __forceinline__ void lds_dma16_sbase(const void *sbase, uint32_t voff, uint32_t lds_byte) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_byte);
  uint32_t saved;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(voff), "s"(sbase)
      : "memory");
}

// LDS byte address of a pointer into a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// 4-byte variant: lane i's 4 bytes land at LDS byte address lds_byte + 4 * i.
__device__ __forceinline__ void lds_dma4_at(const void *gaddr, uint32_t lds_byte) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_byte);
  uint32_t saved;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(gaddr)
      : "memory");
}

// The same load with the LDS destination given as a pointer into a
// __shared__ object.
__device__ __forceinline__ void lds_dma16(const void *gaddr, void *lds_dst_wave) {
  lds_dma16_at(gaddr, lds_addr(lds_dst_wave));
}

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt <= n only.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS traffic only.  __syncthreads() also fences
// global memory, i.e. waits for every outstanding vector-memory operation,
// which would retire loads deliberately kept in flight across the barrier.
// Callers have already waited for the loads the next step reads, so only this
// wave's own LDS operations need to complete before the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Exclusive count of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fminf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace dsa
