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

#include <type_traits>
#include <utility>

#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x by the hardware exponential alone (v_exp_f32).  Results below 2^-126
// come out as zero instead of denormals; softmax terms that small relative
// to the running maximum change nothing, and the range fix-up exp2f adds
// for them costs four vector instructions per call.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// --------------------------------------------------------------------------
// fp32 path (1 <= heads <= 64, d_v <= d_qk <= 256).
//
// A workgroup of 4 waves takes every head of one query row over a range of
// its selected slots, 64 slots (one chunk) at a time, so that each gathered
// row is read from memory once for all heads:
//   * the 64 rows of the chunk go to LDS (zero-filled past d_qk and for
//     slots that select nothing);
//   * logits S = Q K^T from fp32 MFMA 16x16x4 tiles: wave w takes slots
//     16w..16w+15 of the chunk for every 16-head tile;
//   * online softmax (base 2, scale folded in), four threads per head;
//   * O += P V from fp32 MFMA tiles again, wave w owning the 16-column
//     output tiles w, w+4, w+8, w+12.
// A row split over several workgroups writes normalised partials and their
// log-sum-exp; mla_f32_combine_kernel merges them.
// --------------------------------------------------------------------------
constexpr int kF32MaxD = 256;
constexpr int kF32Chunk = 64;
constexpr int kF32Ld = kF32MaxD + 4;      // row stride in floats: 16 rows x 4 columns hit 64 banks
constexpr int kF32PLd = kF32Chunk + 4;

struct MlaF32Lds {
  float q[64][kF32Ld];
  float kv[kF32Chunk][kF32Ld];
  float p[64][kF32PLd];
  float alpha[64];
  float l[64];
  float m[64];
  int64_t row[kF32Chunk];
};

__global__ __launch_bounds__(256) void mla_f32_kernel(BatchDev bt, KeysDev kd, int heads, int d_qk, int d_v,
                                                      const float *__restrict__ q,
                                                      const float *__restrict__ kv,
                                                      const int32_t *__restrict__ idx, int k,
                                                      int slots_per_split, int vec4, float sm_scale,
                                                      float *__restrict__ out, float *__restrict__ lse,
                                                      float *__restrict__ part_o,
                                                      float *__restrict__ part_lse) {
  __shared__ MlaF32Lds sh;
  const int t = blockIdx.x;
  const int sp = blockIdx.y;
  const int nsplit = gridDim.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = seq_of_row(bt, t);
  const int ht_n = (heads + 15) >> 4;          // 16-head tiles
  const int hp = ht_n * 16;
  const int nk = (d_qk + 3) >> 2;              // K steps of the logits
  const int nt_n = (d_v + 15) >> 4;            // 16-column output tiles
  const int s_begin = sp * slots_per_split;
  const int s_end = min(k, s_begin + slots_per_split);
  const int32_t *irow = idx + (int64_t)t * k;

  // queries of every head, zero past d_qk and past the last head
  // (each wave's 16 heads x 4 loads go out before the LDS stores)
  const float *qt = q + (int64_t)t * heads * d_qk;
  {
    float v[16][4];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int h = wave + 4 * i;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = lane + 64 * u;
        v[i][u] = (h < heads && c < d_qk) ? qt[(int64_t)h * d_qk + c] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u) sh.q[wave + 4 * i][lane + 64 * u] = v[i][u];
  }

  const float c2 = sm_scale * kLog2e;
  const int r16 = lane & 15, g4 = lane >> 4;
  float m_run = -INFINITY, l_run = 0.f;        // of head tid >> 2 (four threads each)
  v4f o[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int n = 0; n < 4; ++n) o[a][n] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int c0 = s_begin; c0 < s_end; c0 += kF32Chunk) {
    // slot -> row of the chunk (the previous chunk's P V is done in this wave;
    // the barrier below makes it done in all before rows are overwritten)
    if (tid < kF32Chunk) {
      const int j = c0 + tid;
      const int s = j < s_end ? irow[j] : -1;
      sh.row[tid] = s >= 0 ? key_row(kd, b, s) : -1;
    }
    __syncthreads();
    // gather: wave w fills rows 16w .. 16w+15 (float4 loads when rows are 16-byte aligned)
    // (all 16 rows' loads are issued before the first LDS store)
    if (vec4) {
      float4 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t row = sh.row[16 * wave + i];
        v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row >= 0 && 4 * lane < d_qk) v[i] = *(const float4 *)(kv + row * d_qk + 4 * lane);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) *(float4 *)&sh.kv[16 * wave + i][4 * lane] = v[i];
    } else {
#pragma unroll
      for (int h8 = 0; h8 < 16; h8 += 4) {
        float v[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t row = sh.row[16 * wave + h8 + i];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int c = lane + 64 * u;
            v[i][u] = (row >= 0 && c < d_qk) ? kv[row * d_qk + c] : 0.f;
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int u = 0; u < 4; ++u) sh.kv[16 * wave + h8 + i][lane + 64 * u] = v[i][u];
      }
    }
    __syncthreads();
    // logits of slots 16w .. 16w+15, in base-2 units, -inf where nothing is selected
    const bool live = sh.row[16 * wave + r16] >= 0;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      if (a < ht_n) {
        v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        const float *qa = &sh.q[16 * a + r16][g4];
        const float *kb = &sh.kv[16 * wave + r16][g4];
        int ks = 0;
        for (; ks + 1 < nk; ks += 2) {
          s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[4 * ks], kb[4 * ks], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[4 * ks + 4], kb[4 * ks + 4], s1, 0, 0, 0);
        }
        if (ks < nk) s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[4 * ks], kb[4 * ks], s0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sh.p[16 * a + 4 * g4 + i][16 * wave + r16] = live ? (s0[i] + s1[i]) * c2 : -INFINITY;
      }
    }
    __syncthreads();
    // online softmax: head tid >> 2, slots 16 (tid & 3) .. +15 of the chunk
    {
      const int h = tid >> 2, qq = tid & 3;
      if (h < hp) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *(const float4 *)&sh.p[h][16 * qq + 4 * u];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < 4; ++u) mx = fmaxf(fmaxf(fmaxf(mx, v[u].x), fmaxf(v[u].y, v[u].z)), v[u].w);
        mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
        const float m_new = fmaxf(m_run, mx);
        float alpha = 1.f, sum = 0.f;
        if (m_new != -INFINITY) {
          alpha = exp2f(m_run - m_new);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            v[u].x = exp2f(v[u].x - m_new);
            v[u].y = exp2f(v[u].y - m_new);
            v[u].z = exp2f(v[u].z - m_new);
            v[u].w = exp2f(v[u].w - m_new);
            sum += (v[u].x + v[u].y) + (v[u].z + v[u].w);
          }
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        sum += __shfl_xor(sum, 1, 64);
        sum += __shfl_xor(sum, 2, 64);
        l_run = l_run * alpha + sum;
        m_run = m_new;
#pragma unroll
        for (int u = 0; u < 4; ++u) *(float4 *)&sh.p[h][16 * qq + 4 * u] = v[u];
        if (qq == 0) sh.alpha[h] = alpha;
      }
    }
    __syncthreads();
    // O = alpha O + P V over the chunk's 64 slots
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      if (a < ht_n) {
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = sh.alpha[16 * a + 4 * g4 + i];
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[a][n][i] *= al[i];
        const float *pa = &sh.p[16 * a + r16][g4];
#pragma unroll 4
        for (int ks = 0; ks < kF32Chunk / 4; ++ks) {
          const float av = pa[4 * ks];
          const float *vb = &sh.kv[4 * ks + g4][r16];
#pragma unroll
          for (int n = 0; n < 4; ++n)
            if (wave + 4 * n < nt_n)
              o[a][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, vb[16 * (wave + 4 * n)], o[a][n], 0, 0, 0);
        }
      }
    }
  }

  // totals of each head to LDS, then normalise and write
  if ((tid & 3) == 0 && (tid >> 2) < hp) {
    sh.l[tid >> 2] = l_run;
    sh.m[tid >> 2] = m_run;
  }
  __syncthreads();
  const bool split = nsplit > 1;
  float *dst = split ? part_o + ((int64_t)t * nsplit + sp) * heads * d_v : out + (int64_t)t * heads * d_v;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    if (a < ht_n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 16 * a + 4 * g4 + i;
        if (h < heads) {
          const float lh = sh.l[h];
          const float inv = lh > 0.f ? 1.f / lh : 0.f;
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            const int d = 16 * (wave + 4 * n) + r16;
            if (d < d_v) dst[(int64_t)h * d_v + d] = o[a][n][i] * inv;
          }
        }
      }
    }
  }
  if (tid < heads) {
    const float lh = sh.l[tid];
    const float v = lh > 0.f ? (sh.m[tid] + log2f(lh)) * kLn2 : -INFINITY;
    if (split)
      part_lse[((int64_t)t * nsplit + sp) * heads + tid] = v;
    else if (lse)
      lse[(int64_t)t * heads + tid] = v;
  }
}

// Merges the fp32 partials of the nsplit ranges of each row: a wave per
// (row, head), lanes over the output columns.
__global__ __launch_bounds__(256) void mla_f32_combine_kernel(int heads, int d_v, int nsplit,
                                                              const float *__restrict__ part_o,
                                                              const float *__restrict__ part_lse,
                                                              float *__restrict__ out,
                                                              float *__restrict__ lse) {
  const int t = blockIdx.x;
  const int h = 4 * blockIdx.y + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (h >= heads) return;
  const float *pl = part_lse + (int64_t)t * nsplit * heads + h;
  const float *po = part_o + ((int64_t)t * nsplit * heads + h) * d_v;
  // groups of 8 ranges: their lse and partial loads go out together, the
  // weights follow from the running max
  float mx = -INFINITY, wsum = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < nsplit; i0 += 8) {
    float li[8], v[8][4];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      li[u] = -INFINITY;
      const int i = i0 + u;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[u][e] = 0.f;
      if (i < nsplit) {
        li[u] = pl[(int64_t)i * heads];
        const float *pi = po + (int64_t)i * heads * d_v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (lane + 64 * e < d_v) v[u][e] = pi[lane + 64 * e];
      }
    }
    float gm = mx;
#pragma unroll
    for (int u = 0; u < 8; ++u) gm = fmaxf(gm, li[u]);
    if (gm == -INFINITY) continue;  // nothing selected so far
    const float c = mx == -INFINITY ? 0.f : expf(mx - gm);
    wsum *= c;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= c;
    mx = gm;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (li[u] != -INFINITY) {
        const float w = expf(li[u] - mx);
        wsum += w;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(w, v[u][e], acc[e]);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  float *o = out + ((int64_t)t * heads + h) * d_v;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (lane + 64 * u < d_v) o[lane + 64 * u] = acc[u] * inv;
  if (lse && lane == 0) lse[(int64_t)t * heads + h] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

// --------------------------------------------------------------------------
// bf16 path: d_qk = 576 (512 latent + 64 rotary), d_v = 512.
//
// A workgroup of NW waves takes one query row (wave w owns HT tiles of 16
// heads, so heads = 16*HT*NW) and a contiguous range of at most 2048 of its
// selected slots, processed 32 at a time:
//   * rows: every slot of the range is resolved once (index -> page -> row)
//     into LDS before the tile loop, so the loop issues no dependent loads;
//   * gather: the 32 selected 1152-byte key rows of a tile go straight into
//     LDS with 16-byte global->LDS loads, column-major in 16-byte chunks
//     (chunk c of token t at 512 c + 16 t), two chunk columns a wave-wide
//     load, each lane loading from its own token's row.  A tile is exactly 36
//     wave-wide loads, spread over the waves with the same count for every
//     tile, so a per-wave vmcnt wait retires exactly the tile that is needed
//     next; three (128 heads) or four tile buffers keep the next tiles in
//     flight while one is computed;
//   * S^T[32 tok x 16 heads] = KV_tile[32 x 576] . Q^T[576 x 16] per head
//       tile (16x16x32 bf16 MFMA; the query is the B operand, held in
//       registers for the whole launch; each LDS fragment feeds every head
//       tile of the wave).  Sixteen lanes read one chunk of sixteen tokens:
//       256 contiguous bytes.  A-operand row m of each 16-token half is token
//       tok_of(m) (a fixed permutation, below), the order in which the
//       value reads of the PV product follow the accumulator;
//   * online softmax per head in the exp2 domain.  A head's reference max
//     only moves when a tile's max exceeds it by more than 8 (so the
//     unnormalised terms stay below 2^8); only then are its O rows and
//     denominator rescaled, which keeps the rescale out of the steady state;
//   * O[16 heads x 512] += P[16 x 32] . V[32 x 512] per head tile.  The S^T
//     accumulator of lane (g, head) holds register i = tokens tok_of(4g+i) of
//     each 16-token half, which is the A-operand slot set of the PV product
//     once its K order is permuted to match; V is read in the same order by
//     LDS transpose reads, so P needs no reordering (with 8 waves of 128 heads
//     the PV product is split over output columns instead: every wave's P
//     fragments pass through LDS, in the same lane order).
// With more than one slot range per row (decode: few rows), each range
// writes its normalised output in bf16 plus its lse, merged by mla_combine.
// --------------------------------------------------------------------------
constexpr int kD = 576;
constexpr int kDv = 512;
constexpr int kKs = kD / 32;                   // 18 K-steps of the QK product
constexpr int kKsLat = kDv / 32;               // 16 of them over the latent part
constexpr int kNt = kDv / 16;                  // 32 output dim tiles
constexpr int kBlk = 32;                       // selected tokens per tile
constexpr int kMaxSlots = 2048;                // slots one workgroup resolves
constexpr int kRowBytes = kD * 2;              // 1152
// Tile layout, column-major in 16-byte chunks: chunk c (dims 8c .. 8c+7) of
// token t sits at byte kColBytes * c + 16 * t.  Sixteen lanes reading one
// chunk of sixteen tokens then read 256 contiguous bytes, which LDS serves at
// its full rate; a row-major tile (any row pitch tried) serves that QK operand
// pattern at half the rate.
constexpr int kChunks = kRowBytes / 16;        // 72 chunks a row
constexpr int kColBytes = kBlk * 16;           // 512: one chunk of the 32 tokens
constexpr int kTileBytes = kChunks * kColBytes;  // 36864
constexpr int kTileLoads = kTileBytes / 1024;  // 36 wave-wide 1 KB loads per tile
// Token of A-operand row m (0..15) of a 16-token half of the QK product.  The
// S^T accumulator then holds tokens 4i + rho(g) in lane group g, the order in
// which the P.V product's value reads proceed.
__device__ __forceinline__ int tok_of(int m) { return 4 * (m & 3) + (((m >> 1) & 2) | ((m >> 3) & 1)); }

// f(integral_constant<int, I>) for each I of the sequence, in order (a loop
// whose index must be a compile-time constant, e.g. an immediate offset).
template <int... I, class F>
__device__ __forceinline__ void for_each_index(std::integer_sequence<int, I...>, F &&f) {
  (f(std::integral_constant<int, I>{}), ...);
}
constexpr int kBufs = 4;                       // tile buffers: one computed, three in flight
constexpr float kRefSlack = 8.f;               // log2 headroom above the reference max
#ifndef DSA_QK_AHEAD
#define DSA_QK_AHEAD 2  // K-steps of A fragments read ahead of the QK MFMAs
#endif
#ifndef DSA_PV_AHEAD
#define DSA_PV_AHEAD 3  // V fragments read ahead of the P.V MFMAs
#endif
static_assert(kColBytes * 2 == 1024, "a wave-wide load fills two chunk columns");

struct MlaLds {
  uint8_t tile[kBufs][kTileBytes];
  int32_t rows[kMaxSlots];           // resolved rows of the range (-1: masked slot)
  int32_t full[kMaxSlots / kBlk];    // tile has no masked slot
};

// 128 heads: the P.V product is split over output columns (see the kernel),
// which needs the P fragments, the rescale factors and the denominators in
// LDS; three tile buffers leave the room.  The P exchange has two buffers
// (tiles alternate), so a tile needs one barrier.
constexpr int kBufsSplit = 3;
struct MlaXchg {
  v8bf p[8][64];     // P fragment of each wave's 16 heads, lane by lane
  float alpha[128];  // rescale factor of each head (valid where resc is set)
  int32_t resc[8];   // wave w rescaled its heads in this tile
};
struct MlaLdsSplit {
  uint8_t tile[kBufsSplit][kTileBytes];
  int32_t rows[kMaxSlots];
  int32_t full[kMaxSlots / kBlk];
  MlaXchg x[2];      // exchange buffers of even and odd tiles
  float inv_l[128];  // 1 / denominator of each head
};

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4s lds_v4s;

template <int NW, int HT>
__global__ __launch_bounds__(NW * 64) void mla_bf16_kernel(
    BatchDev bt, KeysDev kd, const __hip_bfloat16 *__restrict__ q,
    const __hip_bfloat16 *__restrict__ kv, const int32_t *__restrict__ idx, int k,
    int slots_per_split, float sm_scale, __hip_bfloat16 *__restrict__ out,
    float *__restrict__ lse, __hip_bfloat16 *__restrict__ part_o, float *__restrict__ part_lse) {
  constexpr int HW = 16 * HT;  // heads per wave
  constexpr int H = HW * NW;
  constexpr int NT = NW * 64;
  // waves below kTileLoads % NW issue one load more per tile than the others
  constexpr int kLHi = (kTileLoads + NW - 1) / NW;
  constexpr int kLLo = kTileLoads / NW;
  // 128 heads: P.V split over output columns -- wave w accumulates every
  // head's output over dims 64w .. 64w+63 -- so each V element is read from
  // LDS by one wave instead of eight (transpose reads run at about 60% of the
  // plain 16-byte read rate); the waves' P fragments go through LDS instead.
  constexpr bool kSplit = NW == 8 && HT == 1;
  constexpr int NB = kSplit ? kBufsSplit : kBufs;  // tile buffers
  constexpr int kOt = kSplit ? kNt / NW : kNt;     // output dim tiles of a wave
  constexpr int kOh = kSplit ? NW : HT;            // output head tiles of a wave
  using Lds = typename std::conditional<kSplit, MlaLdsSplit, MlaLds>::type;
  __shared__ Lds sh;

  const int t = blockIdx.x;
  const int split = blockIdx.y;
  const int nsplit = gridDim.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;    // lane group
  const int n16 = lane & 15;  // column within a 16-wide tile
  const int slot_begin = split * slots_per_split;
  const int slot_end = min(k, slot_begin + slots_per_split);
  const int nslot = max(slot_end - slot_begin, 0);
  const int nblk = (nslot + kBlk - 1) / kBlk;
  const int32_t *idx_t = idx + (int64_t)t * k;
  const uint8_t *kv_bytes = (const uint8_t *)kv;

  // Prologue order: loads whose results are needed first go out first, so
  // that waiting for them leaves the (large) query loads in flight.
  // (1) this thread's selected positions
  constexpr int kPer = kMaxSlots / NT;
  static_assert(kPer * NT == kMaxSlots, "slots split evenly over the threads");
  int sel[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = tid + u * NT;
    sel[u] = i < nslot ? idx_t[slot_begin + i] : -1;
  }
  // (2) first round of a 64-ary search for the row's sequence: lane l reads
  // q_seq_start[l * step]
  const int step0 = (bt.num_seqs + 63) >> 6;
  const int pos0 = lane * step0;
  const int qs0 = pos0 < bt.num_seqs ? bt.q_seq_start[pos0] : 0x7FFFFFFF;
  __builtin_amdgcn_sched_barrier(0);
  // (3) query operand (B of S^T): heads HW*w + 16*ht + n16, dims 32*ks + 8g .. +8
  v8bf qf[HT][kKs];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const __hip_bfloat16 *qh = q + ((int64_t)t * H + HW * wave + 16 * ht + n16) * kD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) qf[ht][ks] = *(const v8bf *)(qh + 32 * ks);
  }
  __builtin_amdgcn_sched_barrier(0);
  // the sequence: the last entry of q_seq_start that is <= t (entries are
  // non-decreasing; the lanes reading such entries form a prefix).  Later
  // rounds only run for more than 64 sequences.  Kept in [0, num_seqs) for
  // any array contents.
  int b = max((int)__popcll(__ballot(qs0 <= t)) - 1, 0) * step0;
  for (int span = min(step0, bt.num_seqs - b); span > 1;) {
    const int step = (span + 63) >> 6;
    const int pos = b + lane * step;
    const bool le = pos < b + span && bt.q_seq_start[pos] <= t;
    const int c = max((int)__popcll(__ballot(le)), 1);
    b += (c - 1) * step;
    span = min(step, span - (c - 1) * step);
  }
  b = __builtin_amdgcn_readfirstlane(b);
  const int64_t row0 = key_row(kd, b, 0);  // stand-in row for masked / pad slots
  // (4) resolve every slot of the range once, and mark the tiles without a
  // masked slot (a wave's 64 slots are two whole tiles)
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = tid + u * NT;
    if (i < nblk * kBlk) sh.rows[i] = sel[u] >= 0 ? (int32_t)key_row(kd, b, sel[u]) : -1;
    const uint64_t valid = __ballot(sel[u] >= 0);
    const int t0 = (64 * wave + u * NT) / kBlk;
    if (lane == 0 && t0 < nblk) sh.full[t0] = (uint32_t)valid == 0xFFFFFFFFu;
    if (lane == 0 && t0 + 1 < nblk) sh.full[t0 + 1] = (uint32_t)(valid >> 32) == 0xFFFFFFFFu;
  }
  lds_barrier();  // LDS only: the query loads stay in flight

  // tile blk -> buffer buf, in 36 wave-wide 1 KB loads: load L fills chunk
  // columns 2L and 2L+1, lane i taking token i % 32, chunk 2L + i / 32 (its
  // 16 bytes land at 16 i of the load's 1 KB, as the layout wants).  A lane's
  // global address is its token's row plus 16 (i / 32), the same for every
  // load of the tile, and load L adds 32 L as an immediate offset.  Wave w
  // issues loads w, w + NW, ...  Masked slots load row0 (their logits are
  // discarded).
  const bool hi = wave < kTileLoads % NW;  // waves that issue kLHi loads a tile
  auto gather = [&](int blk, int buf) __attribute__((always_inline)) {
    const int ln = opaque_lane_id();
    int row = sh.rows[blk * kBlk + (ln & 31)];
    if (row < 0) row = (int)row0;
    const uint8_t *src = kv_bytes + (int64_t)row * kRowBytes + 16 * (ln >> 5) + 32 * wave;
    const uint32_t tb = lds_addr(&sh.tile[buf][0]) + 1024 * wave;
    for_each_index(std::make_integer_sequence<int, kLHi>{}, [&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      if (u < kLLo || hi) lds_dma16_imm<32 * NW * u>(src, tb + 1024 * NW * u);
    });
  };
  // wait until at most `n` tiles of this wave's loads are still in flight
  auto wait_tiles = [&](int n) __attribute__((always_inline)) {
    if (hi) {
      if (n >= 2) wait_vmcnt<(2 * kLHi < 63 ? 2 * kLHi : 63)>();
      else if (n == 1) wait_vmcnt<(kLHi < 63 ? kLHi : 63)>();
      else wait_vmcnt<0>();
    } else {
      if (n >= 2) wait_vmcnt<(2 * kLLo < 63 ? 2 * kLLo : 63)>();
      else if (n == 1) wait_vmcnt<(kLLo < 63 ? kLLo : 63)>();
      else wait_vmcnt<0>();
    }
  };

  // o[a][j]: heads 16a + 4g + i (i < 4) of the wave's head tile a (split:
  // every wave's), dims 16 * (dim tile j) + n16 (split: dim tiles kOt*w + j)
  v4f o[kOh][kOt];
  float m_ref[HT], l_part[HT];  // reference max (log2 domain), this lane's denominator share
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    m_ref[ht] = -INFINITY;
    l_part[ht] = 0.f;
  }
#pragma unroll
  for (int a = 0; a < kOh; ++a)
#pragma unroll
    for (int i = 0; i < kOt; ++i) o[a][i] = v4f{0.f, 0.f, 0.f, 0.f};
  const float zscale = sm_scale * kLog2e;

  // The query loads must be complete (and known complete to the compiler)
  // before the tile loop: otherwise its wait bookkeeping re-waits for them in
  // every iteration, draining the tile loads kept in flight.  They complete
  // together with tile 0's gather; the next tiles go out after.
  // 128 heads fill all NB buffers here and refill a buffer right after the
  // tile's barrier (see below); the others keep one buffer for the gather at
  // the top of each tile.
  constexpr int kAhead = kSplit ? NB : NB - 1;
  if (nblk > 0) gather(0, 0);
  wait_vmcnt<0>();
  for (int p = 1; p < kAhead && p < nblk; ++p) gather(p, p);
  lds_barrier();

  for (int blk = 0; blk < nblk; ++blk) {
    const int buf = blk % NB;
    if (!kSplit && blk + NB - 1 < nblk) gather(blk + NB - 1, (blk + NB - 1) % NB);
    const uint8_t *tile = sh.tile[buf];
    const int32_t *rows = sh.rows + blk * kBlk;

    // ---- S^T = KV . Q^T: tokens 0-15 / 16-31 x each head tile ----
    v4f s0[HT], s1[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      s0[ht] = v4f{0.f, 0.f, 0.f, 0.f};
      s1[ht] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    // A fragments: lane (g, n16) reads chunk 4 ks + g of token tok_of(n16)
    // of each 16-token half (K-steps 16-17 are the rotary dims)
    const uint8_t *abase = tile + kColBytes * g + 16 * tok_of(n16);
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      const v8bf a0 = *(const v8bf *)(abase + 4 * kColBytes * ks);
      const v8bf a1 = *(const v8bf *)(abase + 256 + 4 * kColBytes * ks);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        s0[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ht][ks], s0[ht], 0, 0, 0);
        s1[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ht][ks], s1[ht], 0, 0, 0);
      }
    }
    // keep two K-steps of A fragments (4 reads) ahead of the QK MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * DSA_QK_AHEAD, 1);
#pragma unroll
    for (int i = 0; i < kKs - DSA_QK_AHEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * HT, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * DSA_QK_AHEAD * HT, 1);

    // ---- online softmax (this lane: head n16 of each tile; tokens tok_of(4g+i), 16+tok_of(4g+i)) ----
    // logits in the log2 domain; masked slots (only in tiles that have any)
    // are -inf
    v8bf pf[HT];
    float alpha[HT];
    bool rescale = false;
    float z[HT][8], xl[HT];
    bool moves = false;  // some head's maximum may pass its reference by more than the slack
    if (__builtin_amdgcn_readfirstlane(sh.full[blk])) {
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          z[ht][i] = s0[ht][i] * zscale;
          z[ht][4 + i] = s1[ht][i] * zscale;
        }
    } else {
      bool ok[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ok[i] = rows[tok_of(4 * g + i)] >= 0;
        ok[4 + i] = rows[16 + tok_of(4 * g + i)] >= 0;
      }
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          z[ht][i] = ok[i] ? s0[ht][i] * zscale : -INFINITY;
          z[ht][4 + i] = ok[4 + i] ? s1[ht][i] * zscale : -INFINITY;
        }
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      xl[ht] = z[ht][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) xl[ht] = fmaxf(xl[ht], z[ht][i]);
      moves |= xl[ht] > m_ref[ht] + kRefSlack || m_ref[ht] == -INFINITY;
    }
    // A lane's own maximum decides: only if some lane's tile maximum passes
    // its head's reference by more than the slack (or the head has no
    // reference yet) does the wave take the heads' maxima across its lane
    // groups and move the references.  Otherwise every term is exp2(z - m)
    // with the reference kept, and no value crosses lanes.
    if (__ballot(moves)) {
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        float x = xl[ht];
        x = fmaxf(x, __shfl_xor(x, 16, 64));
        x = fmaxf(x, __shfl_xor(x, 32, 64));
        const float m_new = x > m_ref[ht] + kRefSlack ? x : m_ref[ht];
        alpha[ht] = m_new == m_ref[ht] ? 1.f : fast_exp2(m_ref[ht] - m_new);
        rescale |= alpha[ht] != 1.f;
        m_ref[ht] = m_new;
      }
    } else {
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) alpha[ht] = 1.f;
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      // a head with no reference yet has seen only masked slots: its terms
      // are exp2(-inf) = 0 against any finite stand-in
      const float m = m_ref[ht] == -INFINITY ? 0.f : m_ref[ht];
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = fast_exp2(z[ht][i] - m);
        sum += pv;
        pf[ht][i] = (__bf16)pv;
      }
      l_part[ht] = l_part[ht] * alpha[ht] + sum;
    }
    if constexpr (kSplit) {
      // V fragments of the wave's four dim tiles (transpose reads, as below),
      // read before the barrier: after it no wave reads this tile's buffer,
      // which is refilled at once.  The lane's offset is made opaque in each
      // tile, so the eight reads share one address register (immediate
      // offsets) instead of eight hoisted out of the loop.
      int voff = 16 * tok_of(4 * g + (n16 >> 2)) + kColBytes * ((n16 >> 1) & 1) + 8 * (n16 & 1) +
                 2 * kColBytes * kOt * wave;
      __asm__ volatile("" : "+v"(voff));
      const uint8_t *vrow = tile + voff;
      v8bf vb[kOt];
#pragma unroll
      for (int j = 0; j < kOt; ++j) {
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vrow + 2 * kColBytes * j));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vrow + 256 + 2 * kColBytes * j));
        __builtin_memcpy(&vb[j], &lo, 8);
        __builtin_memcpy((char *)&vb[j] + 8, &hi, 8);
      }
      // this wave's P fragment, rescale flag and factors go to this tile's
      // exchange buffer; after the barrier every wave reads all eight
      MlaXchg &xc = sh.x[blk & 1];
      *(v8bf *)&xc.p[wave][lane] = pf[0];
      const bool any = __ballot(rescale) != 0;
      if (lane == 0) xc.resc[wave] = any;
      if (any) {  // (its address is computed here: a register held across the loop would spill)
        const int ln = opaque_lane_id();
        if (ln < 16) xc.alpha[16 * wave + ln] = alpha[0];
      }
      // One barrier a tile.  Before it: the next tile has landed (this wave's
      // share of it; tile blk+2 may stay in flight).  After it: the next tile
      // and this tile's P are visible to every wave, and every wave is done
      // with this tile's buffer (QK operands and V fragments), which takes
      // tile blk+NB at the top of the next tile.  The exchange
      // buffer is written again for tile blk+2, after the next barrier,
      // which every wave reaches only once its P.V product of this tile has
      // read it.
      wait_tiles(min(nblk - 1, blk + NB - 1) - (blk + 1));
      lds_barrier();
      // This tile's buffer is free: it takes tile blk+NB, whose loads go out
      // one between each two head tiles of the P.V product below (all eight
      // waves issuing their loads at once queue them in the CU's address
      // unit for hundreds of clocks).  The row index is read first, so that
      // its LDS latency passes under the first products.
      const bool refill = blk + NB < nblk;
      int rrow = 0;
      if (refill) rrow = sh.rows[(blk + NB) * kBlk + (opaque_lane_id() & 31)];
      // ---- O[all heads, dims 64w..64w+63] += P . V ----
      // rescales first, behind one wave-uniform branch (rare), so that the
      // products below are one block in which P reads run ahead of the MFMAs
      const v4i rf0 = *(const v4i *)&xc.resc[0], rf1 = *(const v4i *)&xc.resc[4];
      if ((rf0.x | rf0.y | rf0.z | rf0.w | rf1.x | rf1.y | rf1.z | rf1.w) != 0) {
#pragma unroll
        for (int a = 0; a < kOh; ++a) {
          if ((a < 4 ? rf0[a & 3] : rf1[a & 3]) != 0) {
            float r[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) r[i] = xc.alpha[16 * a + 4 * g + i];
#pragma unroll
            for (int j = 0; j < kOt; ++j)
#pragma unroll
              for (int i = 0; i < 4; ++i) o[a][j][i] *= r[i];
          }
        }
      }
      v8bf pa = xc.p[0][lane];
      const uint8_t *rsrc = kv_bytes;
      const uint32_t rtb = lds_addr(&sh.tile[buf][0]) + 1024 * wave;
      for_each_index(std::make_integer_sequence<int, kOh>{}, [&](auto ac) __attribute__((always_inline)) {
        constexpr int a = decltype(ac)::value;
        v8bf pn;
        if (a + 1 < kOh) pn = xc.p[a + 1][lane];  // one head tile ahead
#pragma unroll
        for (int j = 0; j < kOt; ++j) o[a][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb[j], o[a][j], 0, 0, 0);
        if (a + 1 < kOh) pa = pn;
        // refill load u = a - 1 after head tile a (a = 1 .. kLHi)
        constexpr int u = a - 1;
        if constexpr (u >= 0 && u < kLHi) {
          if (refill) {
            if constexpr (u == 0) {
              const int row = rrow < 0 ? (int)row0 : rrow;
              rsrc = kv_bytes + (int64_t)row * kRowBytes + 16 * (opaque_lane_id() >> 5) + 32 * wave;
            }
            if (u < kLLo || hi) lds_dma16_imm<32 * NW * u>(rsrc, rtb + 1024 * NW * u);
          }
        }
      });
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 3);
#pragma unroll
      for (int a = 0; a + 2 < kOh; ++a) {
        __builtin_amdgcn_sched_group_barrier(0x008, kOt, 3);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 3);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * kOt, 3);
    } else {
      if (__ballot(rescale)) {  // O rows of this lane are heads 4g+i of each tile
  #pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          float r[4];
  #pragma unroll
          for (int i = 0; i < 4; ++i) r[i] = __shfl(alpha[ht], 4 * g + i, 64);
  #pragma unroll
          for (int nt = 0; nt < kNt; ++nt)
  #pragma unroll
            for (int i = 0; i < 4; ++i) o[ht][nt][i] *= r[i];
        }
      }

      // ---- O += P . V ----
      // inside a 16-lane group, lane i names 8 bytes of row i/4 (dims 4*(i%4)..+3
      // of a 16-dim tile); the transpose read hands lane i column i of the four
      // rows: 4 consecutive tokens of one dim, the B-operand slot order
      const uint8_t *vrow = tile + 16 * tok_of(4 * g + (n16 >> 2)) + kColBytes * ((n16 >> 1) & 1) + 8 * (n16 & 1);
  #pragma unroll
      for (int nt = 0; nt < kNt; ++nt) {
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vrow + 2 * kColBytes * nt));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vrow + 256 + 2 * kColBytes * nt));
        v8bf vb;
        __builtin_memcpy(&vb, &lo, 8);
        __builtin_memcpy((char *)&vb + 8, &hi, 8);
  #pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          o[ht][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[ht], vb, o[ht][nt], 0, 0, 0);
      }
      // keep three V fragments (6 transpose reads) ahead of the PV MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * DSA_PV_AHEAD, 0);
  #pragma unroll
      for (int i = 0; i < kNt - DSA_PV_AHEAD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, HT, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, DSA_PV_AHEAD * HT, 0);
    }

    if constexpr (!kSplit) {
      // the next tile must have landed; the ones after it may stay in flight
      wait_tiles(min(nblk - 1, blk + NB - 1) - (blk + 1));
      lds_barrier();
    }
  }

  // ---- finish: denominators, output ----
  __hip_bfloat16 *ot = nsplit == 1 ? out + (int64_t)t * H * kDv : part_o + ((int64_t)t * nsplit + split) * H * kDv;
  float *lt_dst = nsplit == 1 ? lse : part_lse + ((int64_t)t * nsplit + split) * H - (int64_t)t * H;
  if constexpr (kSplit) {
    // the wave's heads' 1 / l and lse; then every head's row of the wave's dims
    float lt = l_part[0];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    if (g == 0) {
      sh.inv_l[16 * wave + n16] = lt > 0.f ? 1.f / lt : 0.f;
      if (lt_dst) lt_dst[(int64_t)t * H + 16 * wave + n16] = lt > 0.f ? (m_ref[0] + log2f(lt)) * kLn2 : -INFINITY;
    }
    lds_barrier();
#pragma unroll
    for (int a = 0; a < kOh; ++a) {
      float ir[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ir[i] = sh.inv_l[16 * a + 4 * g + i];
#pragma unroll
      for (int j = 0; j < kOt; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ot[(int64_t)(16 * a + 4 * g + i) * kDv + 16 * (kOt * wave + j) + n16] = __float2bfloat16(o[a][j][i] * ir[i]);
    }
  } else {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float lt = l_part[ht];
      lt += __shfl_xor(lt, 16, 64);
      lt += __shfl_xor(lt, 32, 64);
      // lane n16 holds (m, l) of head HW*w + 16*ht + n16
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse_h = lt > 0.f ? (m_ref[ht] + log2f(lt)) * kLn2 : -INFINITY;
      float ir[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ir[i] = __shfl(inv, 4 * g + i, 64);
      const int h0 = HW * wave + 16 * ht + 4 * g;  // first head of this lane's O rows
#pragma unroll
      for (int nt = 0; nt < kNt; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ot[(int64_t)(h0 + i) * kDv + 16 * nt + n16] = __float2bfloat16(o[ht][nt][i] * ir[i]);
      if (g == 0 && lt_dst) lt_dst[(int64_t)t * H + HW * wave + 16 * ht + n16] = lse_h;
    }
  }
}

// Merge of split partials: lse = log sum_i e^{lse_i}, o = sum_i e^{lse_i - lse} o_i.
// Block = 4 heads x 64 lanes; a lane owns 8 consecutive dims (16-byte loads).
// The split loops are unrolled by 8 so that up to 8 loads are in flight.
constexpr int kMaxSplits = 32;

__global__ __launch_bounds__(256) void mla_combine_kernel(int heads, int nsplit,
                                                          const __hip_bfloat16 *__restrict__ part_o,
                                                          const float *__restrict__ part_lse,
                                                          __hip_bfloat16 *__restrict__ out,
                                                          float *__restrict__ lse) {
  const int t = blockIdx.x;
  const int h = 4 * blockIdx.y + (threadIdx.x >> 6);
  const int d0 = 8 * (threadIdx.x & 63);
  if (h >= heads) return;
  const float *pl = part_lse + (int64_t)t * nsplit * heads + h;
  const __hip_bfloat16 *po = part_o + ((int64_t)t * nsplit * heads + h) * kDv + d0;
  const int64_t pstride = (int64_t)heads * kDv;
  // the partials' loads go out together with their lse loads (one memory
  // round trip per group of 8 splits); the weights follow from the group max
  float mx = -INFINITY, wsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < nsplit; i0 += 8) {
    v8bf v[8];
    float li[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u;
      li[u] = -INFINITY;
      if (i < nsplit) {
        li[u] = pl[(int64_t)i * heads];
        v[u] = *(const v8bf *)(po + i * pstride);
      }
    }
    float gm = mx;
#pragma unroll
    for (int u = 0; u < 8; ++u) gm = fmaxf(gm, li[u]);
    if (gm == -INFINITY) continue;  // nothing selected so far
    // rescale what was accumulated against the previous max
    const float c = mx == -INFINITY ? 0.f : expf(mx - gm);
    wsum *= c;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= c;
    mx = gm;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (i0 + u < nsplit && li[u] != -INFINITY) {
        const float w = expf(li[u] - mx);
        wsum += w;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(w, (float)v[u][j], acc[j]);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  v8bf r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)(acc[j] * inv);
  *(v8bf *)(out + ((int64_t)t * heads + h) * kDv + d0) = r;
  if (lse && d0 == 0) lse[(int64_t)t * heads + h] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

// --------------------------------------------------------------------------
// launchers
// --------------------------------------------------------------------------
// Ranges per fp32 row: enough workgroups to cover the CUs, at least one
// 64-slot chunk each; ranges are whole chunks.
static int mla_f32_chunks_per_split(int num_queries, int k) {
  const int nch = (k + kF32Chunk - 1) / kF32Chunk;
  int s = (256 + num_queries - 1) / num_queries;
  if (s > nch) s = nch;
  if (s < 1) s = 1;
  return (nch + s - 1) / s;
}

int mla_f32_splits(int num_queries, int k) {
  if (num_queries <= 0) return 1;
  const int nch = (k + kF32Chunk - 1) / kF32Chunk;
  const int per = mla_f32_chunks_per_split(num_queries, k);
  return (nch + per - 1) / per;
}

size_t mla_f32_workspace_bytes(int num_queries, int heads, int d_v, int k) {
  const int s = mla_f32_splits(num_queries, k);
  if (s <= 1) return 0;
  const size_t po = ((size_t)num_queries * s * heads * d_v * sizeof(float) + 15) / 16 * 16;
  return po + (size_t)num_queries * s * heads * sizeof(float);
}

size_t mla_f32_workspace_bound(int num_queries, int heads, int d_v) {
  if (num_queries <= 0) return 0;
  const int s = (256 + num_queries - 1) / num_queries;  // no k gives more ranges than this
  if (s <= 1) return 0;
  const size_t po = ((size_t)num_queries * s * heads * d_v * sizeof(float) + 15) / 16 * 16;
  return po + (size_t)num_queries * s * heads * sizeof(float);
}

hipError_t launch_mla_f32(const BatchDev &bt, const KeysDev &kd, int num_queries, int heads,
                          int d_qk, int d_v, const float *q, const float *kv,
                          const int32_t *indices, int k, float sm_scale, float *out, float *lse,
                          void *workspace, hipStream_t stream) {
  if (num_queries == 0) return hipSuccess;
  const int per = mla_f32_chunks_per_split(num_queries, k);
  const int nsplit = mla_f32_splits(num_queries, k);
  float *part_o = nullptr, *part_lse = nullptr;
  if (nsplit > 1) {
    part_o = (float *)workspace;
    part_lse = (float *)((char *)workspace +
                         ((size_t)num_queries * nsplit * heads * d_v * sizeof(float) + 15) / 16 * 16);
  }
  hipLaunchKernelGGL(mla_f32_kernel, dim3(num_queries, nsplit), dim3(256), 0, stream, bt, kd, heads, d_qk,
                     d_v, q, kv, indices, k, per * kF32Chunk, (int)(d_qk % 4 == 0 && (uintptr_t)kv % 16 == 0),
                     sm_scale, out, lse, part_o, part_lse);
  if (nsplit > 1)
    hipLaunchKernelGGL(mla_f32_combine_kernel, dim3(num_queries, (heads + 3) / 4), dim3(256), 0, stream, heads,
                       d_v, nsplit, part_o, part_lse, out, lse);
  return hipGetLastError();
}

int mla_bf16_splits(int num_queries, int heads, int k) {
  (void)heads;
  if (num_queries <= 0) return 1;
  const int min_s = (k + kMaxSlots - 1) / kMaxSlots;  // a range resolves at most 2048 slots
  int s = (256 + num_queries - 1) / num_queries;      // aim for one workgroup per CU
  const int max_s = (k + 4 * kBlk - 1) / (4 * kBlk);  // at least 4 tiles per range
  if (s > max_s) s = max_s;
  if (s < min_s) s = min_s;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : s;
}

size_t mla_bf16_workspace_bytes(int num_queries, int heads, int d_v, int k) {
  const int s = mla_bf16_splits(num_queries, heads, k);
  if (s <= 1) return 0;
  // bf16 partial outputs, then fp32 partial lse (16-byte aligned)
  const size_t po = ((size_t)num_queries * s * heads * d_v * 2 + 15) / 16 * 16;
  return po + (size_t)num_queries * s * heads * sizeof(float);
}

hipError_t launch_mla_bf16(const BatchDev &bt, const KeysDev &kd, int num_queries, int heads,
                           const void *q, const void *kv, const int32_t *indices, int k,
                           float sm_scale, void *out, float *lse, void *workspace,
                           hipStream_t stream) {
  if (num_queries == 0) return hipSuccess;
  const int nsplit = mla_bf16_splits(num_queries, heads, k);
  const int per = ((k + nsplit - 1) / nsplit + kBlk - 1) / kBlk * kBlk;
  if (per > kMaxSlots) return hipErrorInvalidValue;
  __hip_bfloat16 *part_o = nullptr;
  float *part_lse = nullptr;
  if (nsplit > 1) {
    part_o = (__hip_bfloat16 *)workspace;
    const size_t po = ((size_t)num_queries * nsplit * heads * kDv * 2 + 15) / 16 * 16;
    part_lse = (float *)((char *)workspace + po);
  }
  const dim3 grid(num_queries, nsplit);
  switch (heads) {
    case 128:
      hipLaunchKernelGGL((mla_bf16_kernel<8, 1>), grid, dim3(512), 0, stream, bt, kd,
                         (const __hip_bfloat16 *)q, (const __hip_bfloat16 *)kv, indices, k, per,
                         sm_scale, (__hip_bfloat16 *)out, lse, part_o, part_lse);
      break;
    case 32:
      hipLaunchKernelGGL((mla_bf16_kernel<2, 1>), grid, dim3(128), 0, stream, bt, kd,
                         (const __hip_bfloat16 *)q, (const __hip_bfloat16 *)kv, indices, k, per,
                         sm_scale, (__hip_bfloat16 *)out, lse, part_o, part_lse);
      break;
    case 64:
      hipLaunchKernelGGL((mla_bf16_kernel<4, 1>), grid, dim3(256), 0, stream, bt, kd,
                         (const __hip_bfloat16 *)q, (const __hip_bfloat16 *)kv, indices, k, per,
                         sm_scale, (__hip_bfloat16 *)out, lse, part_o, part_lse);
      break;
    case 16:
      hipLaunchKernelGGL((mla_bf16_kernel<1, 1>), grid, dim3(64), 0, stream, bt, kd,
                         (const __hip_bfloat16 *)q, (const __hip_bfloat16 *)kv, indices, k, per,
                         sm_scale, (__hip_bfloat16 *)out, lse, part_o, part_lse);
      break;
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(num_queries, (heads + 3) / 4), dim3(256), 0, stream, heads,
                     nsplit, part_o, part_lse, (__hip_bfloat16 *)out, lse);
  return hipGetLastError();
}

}  // namespace dsa
