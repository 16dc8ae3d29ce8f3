// Sparse MLA over the selected tokens, absorbed (MQA) form (gfx950).
//
// For query row t, head h and the selected positions J of that row:
//   z_s = sm_scale * q[t,h,:] . kv[s,:]       (key row = [c^KV ; k^R], d_qk wide)
//   o[t,h,:] = sum_s softmax_J(z)_s * kv[s, :d_v],   lse[t,h] = log sum_s e^{z_s}
// ("DeepSeek Sparse Attention DSA Architecture Guide": "Stage 2: Fine-Grained
// Token Selection", gather and u_t equations -- the softmax runs over S_t
// only -- with the latent + decoupled-rotary logit of its MLA section; the
// online softmax follows the IO-aware fused-kernel technique of "Sparse
// Attention Architectures for Long-Context Inference", section 5.1.)
// The output stays in latent space (before W_UV).
#include <hip/hip_bf16.h>

#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// --------------------------------------------------------------------------
// fp32 path (heads <= 64, d_qk <= 128, d_v <= d_qk): one wave per (t, h).
// Lanes take 64 selected tokens at a time for the logits; each lane then
// owns output dims lane and lane + 64.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(64) void mla_f32_kernel(BatchDev bt, KeysDev kd, int heads, int d_qk,
                                                     int d_v, const float *__restrict__ q,
                                                     const float *__restrict__ kv,
                                                     const int32_t *__restrict__ idx, int k,
                                                     float sm_scale, float *__restrict__ out,
                                                     float *__restrict__ lse) {
  __shared__ float q_s[128];
  __shared__ float p_s[64];
  __shared__ int64_t row_s[64];
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const int b = seq_of_row(bt, t);
  const float *qh = q + ((int64_t)t * heads + h) * d_qk;
  for (int d = lane; d < d_qk; d += 64) q_s[d] = qh[d];
  __syncthreads();
  float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int j0 = 0; j0 < k; j0 += 64) {
    const int j = j0 + lane;
    const int s = j < k ? idx[(int64_t)t * k + j] : -1;
    float z = -INFINITY;
    int64_t row = -1;
    if (s >= 0) {
      row = key_row(kd, b, s);
      const float *r = kv + row * d_qk;
      float dot = 0.f;
      for (int d = 0; d < d_qk; ++d) dot = fmaf(q_s[d], r[d], dot);
      z = dot * sm_scale;
    }
    const float m_new = fmaxf(m, wave_max(z));
    float p = 0.f, alpha = 1.f;
    if (m_new != -INFINITY) {
      p = s >= 0 ? expf(z - m_new) : 0.f;
      alpha = expf(m - m_new);
    }
    float psum = p;
    for (int off = 32; off > 0; off >>= 1) psum += __shfl_xor(psum, off, 64);
    l = l * alpha + psum;
    acc0 *= alpha;
    acc1 *= alpha;
    m = m_new;
    p_s[lane] = p;
    row_s[lane] = row;
    __syncthreads();
    const int cnt = min(64, k - j0);
    for (int jj = 0; jj < cnt; ++jj) {
      const int64_t r = row_s[jj];
      if (r < 0) continue;
      const float *v = kv + r * d_qk;
      const float pj = p_s[jj];
      if (lane < d_v) acc0 = fmaf(pj, v[lane], acc0);
      if (lane + 64 < d_v) acc1 = fmaf(pj, v[lane + 64], acc1);
    }
    __syncthreads();
  }
  float *o = out + ((int64_t)t * heads + h) * d_v;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (lane < d_v) o[lane] = acc0 * inv;
  if (lane + 64 < d_v) o[lane + 64] = acc1 * inv;
  if (lse && lane == 0) lse[(int64_t)t * heads + h] = l > 0.f ? m + logf(l) : -INFINITY;
}

// --------------------------------------------------------------------------
// bf16 path: d_qk = 576 (512 latent + 64 rotary), d_v = 512, heads = 16*NW.
//
// A workgroup of NW waves takes one query row (all its heads; wave w owns
// heads 16w..16w+15) and a contiguous range of its selected slots.  Slots
// are processed 32 at a time.  The 32 selected 1152-byte key rows are
// gathered straight into an LDS tile with 16-byte global->LDS loads (row
// pitch 1168 bytes to spread LDS banks; the tile is double buffered, so the
// next tile's loads are in flight while the current one is used).  Per wave:
//   S^T[32 tok x 16 heads] = KV_tile[32 x 576] . Q^T[576 x 16]
//       (16x16x32 bf16 MFMA; the query stays in registers as the B operand)
//   online softmax per head on the accumulators (exp2 domain);
//   O[16 heads x 512] += P[16 x 32] . V[32 x 512]
// The S^T accumulator of lane (g, head) holds tokens 4g+i of each 16-token
// half, which is exactly the A-operand slot set of the PV product once the
// K order of that product is permuted to match (tokens 4g..4g+3 and
// 16+4g..16+4g+3 for lane group g); the V operand is read with the same
// permutation, so P never leaves its registers.
// With more than one slot range per row (decode: few rows), each range
// writes a normalised fp32 partial and its lse, merged by mla_combine.
// --------------------------------------------------------------------------
constexpr int kD = 576;
constexpr int kDv = 512;
constexpr int kBlk = 32;                       // selected tokens per tile
constexpr int kRowBytes = kD * 2;              // 1152
constexpr int kRowSlots = kRowBytes / 16 + 1;  // 72 data chunks + 1 pad chunk
constexpr int kRowStride = kRowSlots * 16;     // 1168-byte LDS row pitch
constexpr int kTileSlots = kBlk * kRowSlots;   // 2336 16-byte slots
constexpr int kTileLoads = (kTileSlots + 63) / 64;     // wave-wide loads per tile
constexpr int kTileBytes = kTileLoads * 64 * 16;       // rounded up to whole loads

template <int NW>
struct MlaLds {
  uint8_t tile[2][kTileBytes];
  int32_t valid[2][kBlk];
};

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4s lds_v4s;

template <int NW>
__global__ __launch_bounds__(NW * 64) void mla_bf16_kernel(
    BatchDev bt, KeysDev kd, const __hip_bfloat16 *__restrict__ q,
    const __hip_bfloat16 *__restrict__ kv, const int32_t *__restrict__ idx, int k,
    int slots_per_split, float sm_scale, __hip_bfloat16 *__restrict__ out,
    float *__restrict__ lse, float *__restrict__ part_o, float *__restrict__ part_lse) {
  constexpr int H = NW * 16;
  __shared__ MlaLds<NW> sh;

  const int t = blockIdx.x;
  const int split = blockIdx.y;
  const int nsplit = gridDim.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;    // lane group
  const int n16 = lane & 15;  // column within a 16-wide tile
  const int b = seq_of_row(bt, t);
  const int slot_begin = split * slots_per_split;
  const int slot_end = min(k, slot_begin + slots_per_split);
  const int nblk = slot_end > slot_begin ? (slot_end - slot_begin + kBlk - 1) / kBlk : 0;
  const int32_t *idx_t = idx + (int64_t)t * k;
  const uint8_t *kv_bytes = (const uint8_t *)kv;
  const int64_t row0 = key_row(kd, b, 0);  // stand-in row for masked / pad slots

  // query operand (B of S^T): head 16*wave + n16, dims 32*ks + 8g .. +8
  v8bf qf[kD / 32];
  {
    const __hip_bfloat16 *qh = q + ((int64_t)t * H + 16 * wave + n16) * kD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) qf[ks] = *(const v8bf *)(qh + 32 * ks);
  }

  // Gather of tile `blk` into buffer `buf`: wave-wide load j of wave w fills
  // LDS slots 64*(NW*j + w) .. +63; slot -> (row = slot / 73, chunk = slot % 73),
  // chunk 72 is pitch padding (reloads chunk 0), rows >= 32 are tail padding.
  auto gather = [&](int blk, int buf) {
    for (int j = 0; NW * j + wave < kTileLoads; ++j) {
      const int base = 64 * (NW * j + wave);
      const int slot = base + lane;
      const int r = slot / kRowSlots;
      int c = slot - r * kRowSlots;
      int64_t row = row0;
      if (r < kBlk) {
        const int si = slot_begin + blk * kBlk + r;
        const int s = si < slot_end ? idx_t[si] : -1;
        if (s >= 0) row = key_row(kd, b, s);
      }
      if (c == kRowSlots - 1 || r >= kBlk) c = 0;
      __builtin_amdgcn_global_load_lds((const void *)(kv_bytes + row * kRowBytes + c * 16),
                                       (lds_void *)(&sh.tile[buf][base * 16]), 16, 0, 0);
    }
    if (tid < kBlk) {
      const int si = slot_begin + blk * kBlk + tid;
      sh.valid[buf][tid] = si < slot_end && idx_t[si] >= 0;
    }
  };

  v4f o_acc[kDv / 16];
#pragma unroll
  for (int i = 0; i < kDv / 16; ++i) o_acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max of this lane's head (log2 domain)
  float l_part = 0.f;       // this lane's share of the running denominator
  const float zscale = sm_scale * kLog2e;

  if (nblk > 0) gather(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    const int buf = blk & 1;
    if (blk + 1 < nblk) gather(blk + 1, buf ^ 1);
    const uint8_t *tile = sh.tile[buf];

    // ---- S^T = KV . Q^T for two 16-token halves ----
    v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) {
      const v8bf a0 = *(const v8bf *)(tile + n16 * kRowStride + 64 * ks + 16 * g);
      const v8bf a1 = *(const v8bf *)(tile + (16 + n16) * kRowStride + 64 * ks + 16 * g);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks], s1, 0, 0, 0);
    }

    // ---- online softmax (this lane: head n16, tokens 4g+i and 16+4g+i) ----
    float z[8];
    float zmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = sh.valid[buf][4 * g + i] ? s0[i] * zscale : -INFINITY;
      z[4 + i] = sh.valid[buf][16 + 4 * g + i] ? s1[i] * zscale : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) zmax = fmaxf(zmax, z[i]);
    zmax = fmaxf(zmax, __shfl_xor(zmax, 16, 64));
    zmax = fmaxf(zmax, __shfl_xor(zmax, 32, 64));
    const float m_new = fmaxf(m_run, zmax);
    float alpha = 1.f;
    float p[8];
    if (m_new == -INFINITY) {
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = 0.f;
    } else {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = exp2f(z[i] - m_new);
    }
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) psum += p[i];
    l_part = l_part * alpha + psum;

    // rescale O rows (heads 4g+i of this lane's O tiles) when any max moved
    if (__ballot(alpha != 1.f)) {
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
      for (int nt = 0; nt < kDv / 16; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o_acc[nt][i] *= al[i];
    }

    // ---- O += P . V ----
    v8bf pa;
#pragma unroll
    for (int i = 0; i < 8; ++i) pa[i] = (__bf16)p[i];
    // V operand by LDS transpose reads: inside a 16-lane group, lane i names
    // 8 bytes of row i/4 (dims 4*(i%4)..+3 of the tile's 16); the read hands
    // lane i column i of the four rows, i.e. 4 consecutive tokens of dim i.
    const uint8_t *vrow = tile + (4 * g + (n16 >> 2)) * kRowStride + 8 * (n16 & 3);
#pragma unroll 8
    for (int nt = 0; nt < kDv / 16; ++nt) {
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vrow + 32 * nt));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vrow + 16 * kRowStride + 32 * nt));
      v8bf vb;
      __builtin_memcpy(&vb, &lo, 8);
      __builtin_memcpy((char *)&vb + 8, &hi, 8);
      o_acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o_acc[nt], 0, 0, 0);
    }

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- finish: denominators, output ----
  float l_tot = l_part;
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  // lanes n16 = head hold (m_run, l_tot) of head 16*wave + n16
  const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_head = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  float inv_row[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) inv_row[i] = __shfl(inv_l, 4 * g + i, 64);
  const int h0 = 16 * wave + 4 * g;  // first head of this lane's O rows
  if (nsplit == 1) {
#pragma unroll
    for (int nt = 0; nt < kDv / 16; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out[((int64_t)t * H + h0 + i) * kDv + 16 * nt + n16] =
            __float2bfloat16(o_acc[nt][i] * inv_row[i]);
    if (lse && g == 0) lse[(int64_t)t * H + 16 * wave + n16] = lse_head;
  } else {
    float *po = part_o + ((int64_t)t * nsplit + split) * H * kDv;
#pragma unroll
    for (int nt = 0; nt < kDv / 16; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) po[(int64_t)(h0 + i) * kDv + 16 * nt + n16] = o_acc[nt][i] * inv_row[i];
    if (g == 0) part_lse[((int64_t)t * nsplit + split) * H + 16 * wave + n16] = lse_head;
  }
}

// Merge of split partials: lse = log sum_i e^{lse_i}, o = sum_i e^{lse_i - lse} o_i.
__global__ __launch_bounds__(256) void mla_combine_kernel(int heads, int nsplit,
                                                          const float *__restrict__ part_o,
                                                          const float *__restrict__ part_lse,
                                                          __hip_bfloat16 *__restrict__ out,
                                                          float *__restrict__ lse) {
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  float mx = -INFINITY;
  for (int i = 0; i < nsplit; ++i) mx = fmaxf(mx, part_lse[((int64_t)t * nsplit + i) * heads + h]);
  float wsum = 0.f;
  float wts[16];
  for (int i = 0; i < nsplit; ++i) {
    const float li = part_lse[((int64_t)t * nsplit + i) * heads + h];
    wts[i] = mx == -INFINITY ? 0.f : expf(li - mx);
    wsum += wts[i];
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  for (int d = threadIdx.x; d < kDv; d += 256) {
    float acc = 0.f;
    for (int i = 0; i < nsplit; ++i)
      acc += wts[i] * part_o[(((int64_t)t * nsplit + i) * heads + h) * kDv + d];
    out[((int64_t)t * heads + h) * kDv + d] = __float2bfloat16(acc * inv);
  }
  if (lse && threadIdx.x == 0) lse[(int64_t)t * heads + h] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

// --------------------------------------------------------------------------
// launchers
// --------------------------------------------------------------------------
hipError_t launch_mla_f32(const BatchDev &bt, const KeysDev &kd, int num_queries, int heads,
                          int d_qk, int d_v, const float *q, const float *kv,
                          const int32_t *indices, int k, float sm_scale, float *out, float *lse,
                          hipStream_t stream) {
  if (num_queries == 0) return hipSuccess;
  hipLaunchKernelGGL(mla_f32_kernel, dim3(num_queries, heads), dim3(64), 0, stream, bt, kd, heads,
                     d_qk, d_v, q, kv, indices, k, sm_scale, out, lse);
  return hipGetLastError();
}

int mla_bf16_splits(int num_queries, int heads, int k) {
  (void)heads;
  if (num_queries <= 0) return 1;
  int s = (256 + num_queries - 1) / num_queries;  // aim for one workgroup per CU
  int max_s = (k + 4 * kBlk - 1) / (4 * kBlk);    // at least 4 tiles per split
  if (s > max_s) s = max_s;
  if (s > 16) s = 16;
  return s < 1 ? 1 : s;
}

size_t mla_bf16_workspace_bytes(int num_queries, int heads, int d_v, int k) {
  const int s = mla_bf16_splits(num_queries, heads, k);
  if (s <= 1) return 0;
  return (size_t)num_queries * s * heads * ((size_t)d_v + 1) * sizeof(float);
}

hipError_t launch_mla_bf16(const BatchDev &bt, const KeysDev &kd, int num_queries, int heads,
                           const void *q, const void *kv, const int32_t *indices, int k,
                           float sm_scale, void *out, float *lse, void *workspace,
                           hipStream_t stream) {
  if (num_queries == 0) return hipSuccess;
  const int nsplit = mla_bf16_splits(num_queries, heads, k);
  const int per = ((k + nsplit - 1) / nsplit + kBlk - 1) / kBlk * kBlk;
  float *part_o = nullptr, *part_lse = nullptr;
  if (nsplit > 1) {
    part_o = (float *)workspace;
    part_lse = part_o + (size_t)num_queries * nsplit * heads * kDv;
  }
  const dim3 grid(num_queries, nsplit);
  switch (heads) {
    case 128:
      hipLaunchKernelGGL(mla_bf16_kernel<8>, grid, dim3(512), 0, stream, bt, kd,
                         (const __hip_bfloat16 *)q, (const __hip_bfloat16 *)kv, indices, k, per,
                         sm_scale, (__hip_bfloat16 *)out, lse, part_o, part_lse);
      break;
    case 64:
      hipLaunchKernelGGL(mla_bf16_kernel<4>, grid, dim3(256), 0, stream, bt, kd,
                         (const __hip_bfloat16 *)q, (const __hip_bfloat16 *)kv, indices, k, per,
                         sm_scale, (__hip_bfloat16 *)out, lse, part_o, part_lse);
      break;
    case 16:
      hipLaunchKernelGGL(mla_bf16_kernel<1>, grid, dim3(64), 0, stream, bt, kd,
                         (const __hip_bfloat16 *)q, (const __hip_bfloat16 *)kv, indices, k, per,
                         sm_scale, (__hip_bfloat16 *)out, lse, part_o, part_lse);
      break;
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(num_queries, heads), dim3(256), 0, stream, heads,
                     nsplit, part_o, part_lse, (__hip_bfloat16 *)out, lse);
  return hipGetLastError();
}

}  // namespace dsa
