// Lightning-indexer score kernels (gfx950).
//
// Computes, for every query row t and causal candidate s < n_t,
//   score[t,s] = scale * sq[t] * sk[s] * sum_j w[t,j] * ReLU(q[t,j,:] . k[s,:])
// ("DeepSeek Sparse Attention DSA Architecture Guide", "Stage 1: The
// Lightning Indexer": ReLU score equation, in its multi-head weighted form;
// FP8 operands per item 1 of that section).  The per-token FP8 scales are
// positive, so they factor out of the ReLU and are applied once per score.
// Each FP8 x FP8 product is exact in fp32, but the MFMA does not add the 128
// products of a dot product as a sequence of fp32 roundings: its sum errs by
// up to about 1.5e-4 of sum |q_d k_d| (measured by the MFMA probe), far below
// the indexer's 1e-3 parity bound.  The [T, n, H_I] per-head products only
// ever live in registers.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

// --------------------------------------------------------------------------
// fp32 path (small shapes: h_i <= 64, d_i <= 128).  One thread per (t, s).
// --------------------------------------------------------------------------
constexpr int kIdxF32Threads = 256;

__global__ __launch_bounds__(kIdxF32Threads) void indexer_f32_kernel(
    BatchDev bt, KeysDev kd, int h_i, int d_i, const float *__restrict__ q,
    const float *__restrict__ w, const float *__restrict__ k, float scale,
    float *__restrict__ scores, int64_t ld) {
  __shared__ float q_s[64 * 128];
  __shared__ float w_s[64];
  const int t = blockIdx.y;
  const int b = seq_of_row(bt, t);
  const int n = candidates_of_row(bt, b, t);
  const int s0 = blockIdx.x * kIdxF32Threads;
  if (s0 >= n) return;  // uniform over the block
  const float *qt = q + (int64_t)t * h_i * d_i;
  for (int i = threadIdx.x; i < h_i * d_i; i += kIdxF32Threads) q_s[i] = qt[i];
  if (threadIdx.x < h_i) w_s[threadIdx.x] = w[(int64_t)t * h_i + threadIdx.x];
  __syncthreads();
  const int s = s0 + threadIdx.x;
  if (s >= n) return;
  const float *kr = k + key_row(kd, b, s) * d_i;
  float acc = 0.f;
  for (int j = 0; j < h_i; ++j) {
    float dot = 0.f;
    for (int d = 0; d < d_i; ++d) dot = fmaf(q_s[j * d_i + d], kr[d], dot);
    acc = fmaf(w_s[j], fmaxf(dot, 0.f), acc);
  }
  scores[(int64_t)t * ld + s] = scale * acc;
}

// --------------------------------------------------------------------------
// FP8 E4M3 path, d_i = 128, h_i = 32 * MT: the MFMA tiling both FP8 kernels
// below share.
//
// Per query row, the heads are the M dimension of a 32x32x64 FP8 MFMA and
// 32 keys its N dimension: a wave multiplies the row's [h_i x 128] query
// block (kept in registers) by a [128 x 32] key tile, two K-steps per 32
// heads.  Lane l supplies operand row/column l % 32 and the 32-byte K-slice
// 32 * (l / 32) of each 64-wide K-step, identically for both operands, so the
// products pair matching d.  The accumulator lane holds column l % 32 (its
// key) and rows 8 * (i / 4) + 4 * (l / 32) + i % 4 (its heads); ReLU and the
// head weight are applied there, and the two half-waves' partial sums are
// added with one cross-lane swap.  Key tiles reach the registers through LDS,
// staged by 16-byte global->LDS loads.
// --------------------------------------------------------------------------
constexpr int kIdxThreads = 256;  // 4 waves

// max(x, 0) in one integer max on the bit pattern: a float with the sign bit
// set (negative, -0, or a negative-signed NaN) is a negative int and becomes
// +0; everything else passes unchanged.
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// x of this lane plus x of the lane 32 away, by a swap of the two half-waves'
// registers (no LDS traffic, unlike a shuffle): both halves get low + high.
__device__ __forceinline__ float add_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}


// --------------------------------------------------------------------------
// FP8 E4M3 path for many query rows per sequence (prefill, chunked prefill).
//
// A workgroup of 4 waves takes QT = 4*QW consecutive query rows of one
// sequence (wave w owns rows QW*w .. QW*w+QW-1) and a block of up to 2048 of
// that sequence's keys, so every key byte crosses L2 once per workgroup
// rather than once per query row.  The block arrives in 128-key stages
// (16 KB of keys, laid out as in the decode form below, plus their fp32
// scales) by global->LDS loads, four buffers deep: three stages are in
// flight while one is scored.  Per wave and 32-key subtile the staged
// fragments feed QW rows x MT head tiles of 32x32x64 MFMAs; ReLU, head
// weights and the head sum happen on the accumulators as in the decode form.
// Keys at or beyond a row's candidate count are computed (the tile is shared)
// but not stored; subtiles beyond every row's count are skipped.
//
// Wait accounting.  Vector-memory stores share the load counter and may
// retire out of order with respect to loads, so each wait allows only as many
// outstanding operations as there are stage loads issued after the stage it
// needs (stores can then only make it wait longer).  The scores of a stage
// are stored at the start of the next one, so by the time of that stage's
// wait they have normally retired and do not eat into the allowance.  Every
// row's scores go out through a buffer store whose range ends at the row's
// last stored key: out-of-range lanes are dropped by the hardware, which
// keeps the store count of every stage the same.
// --------------------------------------------------------------------------
constexpr int kTStageKeys = 128;
constexpr int kTStageBytes = kTStageKeys * 128;     // 16 KB
constexpr int kTStageLoads = kTStageBytes / 1024;   // 16 wave-wide key loads per stage
constexpr int kTBufs = 4;
constexpr int kTKeysPerBlock = 2048;
constexpr int kTPages = kTKeysPerBlock / kPageSize;

// Chunk permutation of a staged 128-byte key row: LDS chunk position p of key
// r holds the key's chunk p ^ kswz(r).  A B-fragment read takes one 16-byte
// chunk from each of 16 consecutive keys per 256-byte bank window; keys of
// one parity share a 128-byte half of that window, and (r >> 1) & 7 gives the
// eight keys of each parity eight distinct chunk positions, so the 16 reads
// cover all banks.
__device__ __forceinline__ int kswz(int r) { return (r >> 1) & 7; }

struct IdxTiledLds {
  uint8_t keys[kTBufs][kTStageBytes];
  float ksc[kTBufs][kTStageKeys];
  int64_t page_row[kTPages];  // flat row of key 64p of the block
};

// Scores of one 32-key subtile of a staged stage for the QW rows of a wave:
// lane key r (= 32*subtile + col), both half-waves end with the full sum.
// The B fragments of key r: K-step ks holds its chunks 4ks + 2*half and
// 4ks + 2*half + 1.  Every row is scored (a row past its candidate count
// only on the causal diagonal; callers drop those), so that the MFMAs of one
// row can overlap the ReLU/weight sum of another.
template <int MT, int QW>
__device__ __forceinline__ void score_subtile(const uint8_t *stage_keys, const float *stage_ksc, int r, int half,
                                              const v8i (&a)[QW][MT][2], const float (&wr)[QW][MT][16],
                                              const float (&row_scale)[QW], float (&out)[QW]) {
  const uint8_t *kb = stage_keys + r * 128;
  v8i bk[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int c = 4 * ks + 2 * half;
    const v4i lo = *(const v4i *)(kb + 16 * (c ^ kswz(r)));
    const v4i up = *(const v4i *)(kb + 16 * ((c + 1) ^ kswz(r)));
    bk[ks] = v8i{lo.x, lo.y, lo.z, lo.w, up.x, up.y, up.z, up.w};
  }
  const float ksc = stage_ksc[r];
  v16f acc[QW][MT];
#pragma unroll
  for (int j = 0; j < QW; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[j][mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j][mt][0], bk[0], v16f{}, 0, 0, 0, 127, 0, 127);
      acc[j][mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j][mt][1], bk[1], acc[j][mt], 0, 0, 0, 127, 0, 127);
    }
#pragma unroll
  for (int j = 0; j < QW; ++j) {
    float sum = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) sum = fmaf(wr[j][mt][i], relu(acc[j][mt][i]), sum);
    sum = add_halves(sum);
    out[j] = sum * row_scale[j] * ksc;
  }
}

template <int MT, int QW, bool PAGED>
__global__ __launch_bounds__(kIdxThreads) void indexer_fp8_tiled_kernel(
    BatchDev bt, KeysDev kd, const uint8_t *__restrict__ q, const float *__restrict__ q_scale,
    const float *__restrict__ w, const uint8_t *__restrict__ k,
    const float *__restrict__ k_scale, float scale, float *__restrict__ scores, int64_t ld) {
  constexpr int H = 32 * MT;
  constexpr int QT = 4 * QW;
  constexpr int kSub = kTStageKeys / 32;  // subtiles per stage
  __shared__ IdxTiledLds sh;

  const int b = blockIdx.z;
  const int q0 = bt.q_seq_start[b];
  const int nq = bt.q_seq_start[b + 1] - q0;
  const int g0 = blockIdx.y * QT;  // first query of the group within the sequence
  if (g0 >= nq) return;
  const int kl = bt.k_len[b];
  const int first_pos = kl - nq;  // position of the sequence's query 0
  const int n_max = first_pos + min(nq, g0 + QT);  // candidates of the group's last row
  const int s_begin = blockIdx.x * kTKeysPerBlock;
  if (s_begin >= n_max) return;
  const int s_end = min(n_max, s_begin + kTKeysPerBlock);
  const int nst = (s_end - s_begin + kTStageKeys - 1) / kTStageKeys;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  // rows of this wave: candidates n, query operand, head weights, output range
  int row_n[QW];
  v8i a[QW][MT][2];
  float wr[QW][MT][16];
  float row_scale[QW];
  __amdgpu_buffer_rsrc_t orow[QW];
#pragma unroll
  for (int j = 0; j < QW; ++j) {
    const int i = g0 + QW * wave + j;
    const bool live = i < nq;
    const int t = q0 + (live ? i : nq - 1);
    row_n[j] = live ? first_pos + i + 1 : 0;
    const uint8_t *qt = q + (int64_t)t * H * 128;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        a[j][mt][ks] = *(const v8i *)(qt + (32 * mt + col) * 128 + 64 * ks + 32 * half);
    const float *wt = w + (int64_t)t * H;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 v = *(const float4 *)(wt + 32 * mt + 8 * r4 + 4 * half);
        wr[j][mt][4 * r4 + 0] = v.x;
        wr[j][mt][4 * r4 + 1] = v.y;
        wr[j][mt][4 * r4 + 2] = v.z;
        wr[j][mt][4 * r4 + 3] = v.w;
      }
    row_scale[j] = q_scale[t] * scale;
    // stored keys of the row: [s_begin, min(n, s_end)); byte offsets from key s_begin
    const int lim = max(min(row_n[j], s_end) - s_begin, 0);
    orow[j] = __builtin_amdgcn_make_buffer_rsrc(scores + (int64_t)t * ld + s_begin, 0, 4 * lim, 0x00020000);
  }
  if (PAGED && tid < kTPages) {
    const int s = min(s_begin + kPageSize * tid, n_max - 1);
    sh.page_row[tid] = key_row(kd, b, s & ~(kPageSize - 1));
  }
  const int64_t kbase = PAGED ? 0 : kd.k_seq_start[b];
  // flat row of key s of the sequence (paged: through the block's page bases)
  auto row_of = [&](int s) __attribute__((always_inline)) -> int64_t {
    if constexpr (PAGED) return sh.page_row[(s - s_begin) >> kPageShift] + (s & (kPageSize - 1));
    else return kbase + s;
  };
  // The query, weight and page loads must be complete (and known complete
  // to the compiler) before the stage loads are issued: otherwise its wait
  // bookkeeping would later wait for them behind stage loads kept in flight.
  // (The barrier alone does not wait for global loads.)
  wait_vmcnt<0>();
  __syncthreads();

  const uint32_t keys0 = __builtin_amdgcn_readfirstlane(lds_addr(&sh.keys[0][0]));
  const uint32_t ksc0 = __builtin_amdgcn_readfirstlane(lds_addr(&sh.ksc[0][0]));
  // stage si -> buffer si % 4.  Key load j (wave + 4m) covers keys 8j .. 8j+7
  // of the stage: lane i stores chunk i % 8 of key 8j + i/8, which holds the
  // key's chunk (i % 8) ^ kswz(key).  Waves 0 and 1 also load the scales of
  // keys 64*wave .. +63.  Keys past n_max reload key n_max - 1.
  auto stage = [&](int si) __attribute__((always_inline)) {
    const int buf = si % kTBufs;
    const int s_stage = s_begin + si * kTStageKeys;
#pragma unroll
    for (int m = 0; m < kTStageLoads / 4; ++m) {
      const int j = wave + 4 * m;
      const int r = 8 * j + (lane >> 3);
      const int s = min(s_stage + r, n_max - 1);
      const int64_t row = row_of(s);
      lds_dma16_at(k + row * 128 + 16 * ((lane & 7) ^ kswz(r)), keys0 + buf * kTStageBytes + 1024 * j);
    }
    if (wave < 2) {
      const int s = min(s_stage + 64 * wave + lane, n_max - 1);
      const int64_t row = row_of(s);
      lds_dma4_at(k_scale + row, ksc0 + buf * (kTStageKeys * 4) + 256 * wave);
    }
  };
  constexpr int kLoads = kTStageLoads / 4;  // key loads per wave per stage (+1 for waves 0, 1)
  // wait until at most `o` stage load groups issued after the needed stage
  // may be in flight
  auto wait_stages = [&](int o) __attribute__((always_inline)) {
    if (wave < 2) {
      if (o >= 2) wait_vmcnt<2 * (kLoads + 1)>(); else if (o == 1) wait_vmcnt<kLoads + 1>(); else wait_vmcnt<0>();
    } else {
      if (o >= 2) wait_vmcnt<2 * kLoads>(); else if (o == 1) wait_vmcnt<kLoads>(); else wait_vmcnt<0>();
    }
  };
  static_assert(kTBufs == 4, "the waits above cover at most two later stages");

  // scores of the previous stage, stored at the start of the next one
  float held[QW][kSub];
  int held_off = 0;  // byte offset of the held stage's key 0 from key s_begin
  auto store_held = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < QW; ++j)
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(held[j][sub]), orow[j],
                                              half ? 0x7FFFFFF0 : held_off + 4 * (32 * sub + col), 0, 0);
  };

  // stages 0 .. 2 in flight, then wait for stage 0
  for (int i = 0; i < kTBufs - 1 && i < nst; ++i) stage(i);
  wait_stages(min(kTBufs - 2, nst - 1));
  lds_barrier();

  for (int si = 0; si < nst; ++si) {
    const int buf = si % kTBufs;
    if (si > 0) store_held();
    if (si + kTBufs - 1 < nst) stage(si + kTBufs - 1);
    const int s_stage = s_begin + si * kTStageKeys;
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) {
      const int sk0 = s_stage + 32 * sub;
      bool any = false;
#pragma unroll
      for (int j = 0; j < QW; ++j) any |= sk0 < row_n[j];
#pragma unroll
      for (int j = 0; j < QW; ++j) held[j][sub] = 0.f;
      if (!any) continue;  // uniform over the wave
      float sc[QW];
      score_subtile<MT, QW>(sh.keys[buf], sh.ksc[buf], 32 * sub + col, half, a, wr, row_scale, sc);
#pragma unroll
      for (int j = 0; j < QW; ++j) held[j][sub] = sc[j];
    }
    held_off = 4 * (si * kTStageKeys);
    // the next stage must have landed; later ones may stay in flight
    wait_stages(min(si + kTBufs - 1, nst - 1) - (si + 1));
    lds_barrier();
  }
  store_held();
}

// --------------------------------------------------------------------------
// Fused indexer -> top-k (prefill; contiguous keys, or paged histories of up
// to kFusedMaxPages pages).
//
// The top-k of a row is the top-k of the union of any partition of its keys,
// because every score depends on one key only ("DeepSeek Sparse Attention DSA
// Architecture Guide", "Stage 1: The Lightning Indexer", item 3).  A
// workgroup takes QT = 4*QW rows of one sequence and streams ALL their keys,
// in ascending position, through the staging of the tiled kernel above; the
// scores are computed by the same code, so they are bit-identical to the
// ones that kernel stores.  Instead of storing them, each row keeps a
// candidate list in the workspace: (score, position) of every key whose
// score beats the row's threshold tau, in ascending position.  Because keys
// arrive in ascending position, a later key equal to tau can never displace
// an earlier one (ties go to the lowest position), so the test is strict.
// When a list could overflow its capacity, the wave that owns the row
// selects the k best entries (score descending, position ascending) and
// compacts them in place, in order; tau becomes the k-th score.  After the
// last key the same selection writes the row's positions, ascending, to the
// output, padded with -1 when the row has fewer than k keys.
//
// Selection (one wave, the row's list in global memory): an exact radix
// select over order-preserving uint32 keys, four 8-bit digits from the top,
// with a 256-bin LDS histogram per pass, gives tau and how many entries equal
// to tau are kept (the first ones in list order); one ordered pass then keeps
// the entries above tau and those first equal ones, with ballot prefix counts
// for the write positions.
// --------------------------------------------------------------------------
// Paged keys: the page of every 64 keys a workgroup streams, resolved into
// LDS before the loop (4 bytes a page), so histories of up to
// fused_topk_max_paged_keys keys.
constexpr int kFusedMaxPages = fused_topk_max_paged_keys / kPageSize;

template <bool PAGED>
struct IdxFusedLds {
  uint8_t keys[kTBufs][kTStageBytes];
  float ksc[kTBufs][kTStageKeys];
  uint32_t hist[4][256];  // one radix histogram per wave
  int32_t want[2][4];     // wave w has a list near full (by stage parity)
  int32_t page[PAGED ? kFusedMaxPages : 1];
};

// Exclusive prefix over the wave's lanes, and wave total, of c in [0, 7].
__device__ __forceinline__ void lane_prefix3(int c, int &before, int &total) {
  before = 0;
  total = 0;
#pragma unroll
  for (int bit = 0; bit < 3; ++bit) {
    const uint64_t m = __ballot((c >> bit) & 1);
    before += lanes_below(m) << bit;
    total += __popcll(m) << bit;
  }
}

// Key (score order) and position of candidate i of a list, 4 per lane.
__device__ __forceinline__ void load_cands(const float *cs, int n, int i, uint32_t (&key)[4], bool (&valid)[4]) {
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (i + 3 < n) {
    v = *(const float4 *)(cs + i);
  } else {
    if (i < n) v.x = cs[i];
    if (i + 1 < n) v.y = cs[i + 1];
    if (i + 2 < n) v.z = cs[i + 2];
  }
  const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    valid[e] = i + e < n;
    key[e] = float_key(f[e]);
  }
}

// The k-th largest key among the n (> k) candidates of a list, and how many
// candidates equal to it belong to the k best.  Every key lies in [lo, hi]
// (bounds uniform over the wave), so the bits above the highest one where lo
// and hi differ are common to every key and are decided before any pass; the
// rest are resolved by radix passes of 8 bits from the top (a list's keys
// share their leading bits, so this saves passes and spreads the first
// digit over the histogram instead of piling it onto one bin).  Each pass
// issues the loads of U chunks of 256 candidates before it uses them.  Whole
// wave; uniform results.
// With `bound` set, only the first digit is resolved: tau is the lowest key of
// the digit that holds the k-th (a lower bound on the k-th key), need_eq is
// -1, and *bound receives how many keys are at least tau.
template <int U>
__device__ void wave_select_kth(const float *cs, int n, int k, uint32_t lo, uint32_t hi, uint32_t *hist,
                                uint32_t &tau, int &need_eq, int *bound = nullptr) {
  const int lane = lane_id();
  if (lo == hi) {  // every key equal: the first k in list order
    tau = lo;
    need_eq = k;
    return;
  }
  const int top = 31 - __builtin_clz(lo ^ hi);  // highest bit where keys may differ
  uint32_t pmask = top == 31 ? 0u : ~0u << (top + 1);
  uint32_t prefix = lo & pmask;
  int need = k;
  for (int hb = top; hb >= 0; hb -= 8) {  // digit: bits hb .. shift
    const int shift = hb >= 7 ? hb - 7 : 0;
    const uint32_t dmask = (2u << (hb - shift)) - 1u;
#pragma unroll
    for (int q = 0; q < 4; ++q) hist[lane + 64 * q] = 0u;
    for (int i0 = 0; i0 < n; i0 += 256 * U) {
      uint32_t key[U][4];
      bool valid[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u) load_cands(cs, n, i0 + 256 * u + 4 * lane, key[u], valid[u]);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (valid[u][e] && (key[u][e] & pmask) == prefix) atomicAdd(&hist[(key[u][e] >> shift) & dmask], 1u);
    }
    // lane l holds bins 255-4l .. 252-4l; scan them from the top
    int c[4], sl = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = (int)hist[255 - 4 * lane - q];
      sl += c[q];
    }
    int incl = sl;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const uint64_t hit = __ballot(incl >= need);
    const int L = hit ? __ffsll((unsigned long long)hit) - 1 : 63;  // empty only on NaN scores
    int acc = incl - sl, digit = 255 - 4 * lane - 3;
    bool found = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (!found && acc + c[q] >= need) {
        digit = 255 - 4 * lane - q;
        found = true;
      } else if (!found) {
        acc += c[q];
      }
    }
    digit = __shfl(digit, L, 64);
    acc = __shfl(acc, L, 64);
    if (bound) {
      *bound = acc + (int)hist[digit];
      tau = prefix | (uint32_t)digit << shift;
      need_eq = -1;
      return;
    }
    need -= acc;
    prefix |= (uint32_t)digit << shift;
    pmask |= dmask << shift;
  }
  tau = prefix;
  need_eq = need;
}

template <int MT, int QW, bool PAGED>
__global__ __launch_bounds__(kIdxThreads) void indexer_topk_fused_kernel(
    BatchDev bt, KeysDev kd, const uint8_t *__restrict__ q,
    const float *__restrict__ q_scale, const float *__restrict__ w, const uint8_t *__restrict__ k,
    const float *__restrict__ k_scale, float scale, int topk, int cap, float *__restrict__ cand_s,
    int32_t *__restrict__ cand_i, int32_t *__restrict__ indices) {
  constexpr int H = 32 * MT;
  constexpr int QT = 4 * QW;
  constexpr int kSub = kTStageKeys / 32;
  __shared__ IdxFusedLds<PAGED> sh;

  const int b = blockIdx.y;
  const int q0 = bt.q_seq_start[b];
  const int nq = bt.q_seq_start[b + 1] - q0;
  const int ngroups = (nq + QT - 1) / QT;
  if ((int)blockIdx.x >= ngroups) return;
  const int g0 = (ngroups - 1 - (int)blockIdx.x) * QT;  // longest rows first
  const int kl = bt.k_len[b];
  const int first_pos = kl - nq;
  const int n_max = first_pos + min(nq, g0 + QT);
  const int nst = (n_max + kTStageKeys - 1) / kTStageKeys;
  const int64_t kbase = PAGED ? 0 : kd.k_seq_start[b];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  int row_t[QW], row_n[QW];
  v8i a[QW][MT][2];
  float wr[QW][MT][16];
  float row_scale[QW];
#pragma unroll
  for (int j = 0; j < QW; ++j) {
    const int i = g0 + QW * wave + j;
    const bool live = i < nq;
    const int t = q0 + (live ? i : nq - 1);
    row_t[j] = t;
    row_n[j] = live ? first_pos + i + 1 : 0;
    const uint8_t *qt = q + (int64_t)t * H * 128;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        a[j][mt][ks] = *(const v8i *)(qt + (32 * mt + col) * 128 + 64 * ks + 32 * half);
    const float *wt = w + (int64_t)t * H;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 v = *(const float4 *)(wt + 32 * mt + 8 * r4 + 4 * half);
        wr[j][mt][4 * r4 + 0] = v.x;
        wr[j][mt][4 * r4 + 1] = v.y;
        wr[j][mt][4 * r4 + 2] = v.z;
        wr[j][mt][4 * r4 + 3] = v.w;
      }
    row_scale[j] = q_scale[t] * scale;
  }
  if constexpr (PAGED) {  // the launcher admits only histories of at most kFusedMaxPages pages
    const int npages = min((n_max + kPageSize - 1) >> kPageShift, kFusedMaxPages);
    for (int p = tid; p < npages; p += kIdxThreads) sh.page[p] = kd.page_table[(int64_t)b * kd.stride + p];
  }
  // (the barrier alone does not wait for global loads)
  wait_vmcnt<0>();
  __syncthreads();

  // flat row of key s of the sequence
  auto row_of = [&](int s) __attribute__((always_inline)) -> int64_t {
    if constexpr (PAGED) return ((int64_t)sh.page[s >> kPageShift] << kPageShift) + (s & (kPageSize - 1));
    else return kbase + s;
  };
  const uint32_t keys0 = __builtin_amdgcn_readfirstlane(lds_addr(&sh.keys[0][0]));
  const uint32_t ksc0 = __builtin_amdgcn_readfirstlane(lds_addr(&sh.ksc[0][0]));
  auto stage = [&](int si) __attribute__((always_inline)) {
    const int buf = si % kTBufs;
    const int s_stage = si * kTStageKeys;
#pragma unroll
    for (int m = 0; m < kTStageLoads / 4; ++m) {
      const int j = wave + 4 * m;
      const int r = 8 * j + (lane >> 3);
      const int64_t row = row_of(min(s_stage + r, n_max - 1));
      lds_dma16_at(k + row * 128 + 16 * ((lane & 7) ^ kswz(r)), keys0 + buf * kTStageBytes + 1024 * j);
    }
    if (wave < 2) {
      const int64_t row = row_of(min(s_stage + 64 * wave + lane, n_max - 1));
      lds_dma4_at(k_scale + row, ksc0 + buf * (kTStageKeys * 4) + 256 * wave);
    }
  };
  constexpr int kLoads = kTStageLoads / 4;
  auto wait_stages = [&](int o) __attribute__((always_inline)) {
    if (wave < 2) {
      if (o >= 2) wait_vmcnt<2 * (kLoads + 1)>(); else if (o == 1) wait_vmcnt<kLoads + 1>(); else wait_vmcnt<0>();
    } else {
      if (o >= 2) wait_vmcnt<2 * kLoads>(); else if (o == 1) wait_vmcnt<kLoads>(); else wait_vmcnt<0>();
    }
  };

  // candidate lists of this wave's rows
  int cnt[QW];
  uint32_t tau[QW];
  float tau_f[QW];  // the score whose key is tau (-inf while tau is 0)
  uint32_t klo[QW], khi[QW];  // this lane's bounds on the keys it appended (the list's: their wave min / max)
#pragma unroll
  for (int j = 0; j < QW; ++j) {
    cnt[j] = 0;
    tau[j] = 0u;  // below every finite score's key
    tau_f[j] = -INFINITY;
    klo[j] = 0xFFFFFFFFu;
    khi[j] = 0u;
  }

  // keep the k best of row j's list (final: write their positions to the
  // output instead, -1 padded)
  auto select = [&](int j, bool final) __attribute__((always_inline)) {
    float *cs = cand_s + (int64_t)row_t[j] * cap;
    int32_t *ci = cand_i + (int64_t)row_t[j] * cap;
    int32_t *out = indices + (int64_t)row_t[j] * topk;
    const int n = cnt[j];
    __threadfence_block();  // the list's stores by every lane of this wave are visible
    const bool all = n <= topk;
    uint32_t th = 0u;
    int need_eq = 0;
    if (!all) {
      uint32_t lo = klo[j], hi = khi[j];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, off, 64));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, off, 64));
      }
      // A compaction needs only a lower bound on the k-th key: it keeps every
      // key of the first digit's boundary bin and above (at least k; later
      // appends must beat the bound, and the final selection is exact).  When
      // that bin holds too many keys to free half the list, it selects exactly.
      int kept_bound = 0;
      wave_select_kth<4>(cs, n, topk, lo, hi, sh.hist[wave], th, need_eq, final ? nullptr : &kept_bound);
      if (!final && need_eq < 0) {
        if (th > 0u && kept_bound <= cap / 2) {
          th -= 1u;  // keep every key > th, i.e. at least the bin's lowest
          need_eq = 0;
        } else {
          wave_select_kth<4>(cs, n, topk, lo, hi, sh.hist[wave], th, need_eq);
        }
      }
    }
    int kept = 0, eq_seen = 0;
    for (int i0 = 0; i0 < n; i0 += 256) {
      const int i = i0 + 4 * lane;
      uint32_t key[4];
      bool valid[4];
      load_cands(cs, n, i, key, valid);
      int idx[4];
      if (i + 3 < n) {  // a whole chunk: one 16-byte load
        const int4 v = *(const int4 *)(ci + i);
        idx[0] = v.x;
        idx[1] = v.y;
        idx[2] = v.z;
        idx[3] = v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) idx[e] = valid[e] ? ci[i + e] : -1;
      }
      // (a compaction writes back the score of each key: equal to the
      // stored one except that -0 becomes +0, which no key comparison tells
      // apart)
      float val[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) val[e] = key_float(key[e]);
      bool gt[4], eq[4];
      int ce = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gt[e] = valid[e] && (all || key[e] > th);
        eq[e] = valid[e] && !all && key[e] == th;
        ce += eq[e];
      }
      int pe, te;
      lane_prefix3(ce, pe, te);
      bool keep[4];
      int run = eq_seen + pe, ck = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        keep[e] = gt[e] || (eq[e] && run < need_eq);
        run += eq[e];
        ck += keep[e];
      }
      int pk, tk;
      lane_prefix3(ck, pk, tk);
      int pos = kept + pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (keep[e]) {
          if (final) {
            out[pos] = idx[e];
          } else {
            cs[pos] = val[e];
            ci[pos] = idx[e];
          }
          ++pos;
        }
      }
      kept += tk;
      eq_seen += te;
    }
    if (final) {
      for (int p = kept + lane; p < topk; p += 64) out[p] = -1;
    } else {
      __threadfence_block();
      cnt[j] = kept;
      tau[j] = th;
      tau_f[j] = key_float(th);
      klo[j] = th;  // every kept key is at least the k-th
    }
  };

  // scores of the previous stage: appended to the lists at the start of the next one
  float held[QW][kSub];
  int held_s0 = 0;  // position of the held stage's key 0
  // A compaction holds up the other waves at the next stage barrier, so the
  // waves compact together: before each barrier a wave flags whether one of
  // its lists would fill within two stages, and after it, if any wave did,
  // every wave compacts each of its lists that is over two thirds full (the
  // waits then overlap).  A list that could overflow in this stage is compacted
  // in any case.  `flags` is the stage parity the flags were written under.
  auto emit_held = [&](int flags) __attribute__((always_inline)) {
    const v4i wf = *(const v4i *)&sh.want[flags][0];
    const bool together = (wf.x | wf.y | wf.z | wf.w) != 0;
#pragma unroll
    for (int j = 0; j < QW; ++j) {
      if (held_s0 >= row_n[j]) continue;  // uniform
      if (cnt[j] + kTStageKeys > cap || (together && 3 * cnt[j] > 2 * cap)) select(j, false);
      float *cs = cand_s + (int64_t)row_t[j] * cap;
      int32_t *ci = cand_i + (int64_t)row_t[j] * cap;
      // A stage wholly inside the row's history skips the per-key position
      // test.  Both half-waves hold every subtile's sums, so subtiles go in
      // pairs: lanes 0-31 take subtile 2p, lanes 32-63 subtile 2p+1, whose
      // keys all follow, so the ballot order is still position order.
      auto append = [&](auto whole) __attribute__((always_inline)) {
#pragma unroll
        for (int sp = 0; sp < kSub / 2; ++sp) {
          const float hv = half ? held[j][2 * sp + 1] : held[j][2 * sp];
          const int s = held_s0 + 32 * (2 * sp + half) + col;
          // key > tau, compared as floats: the key order is the order of the
          // (finite) scores with -0 equal to +0, which float comparison keeps
          const bool ok = (decltype(whole)::value || s < row_n[j]) && hv > tau_f[j];
          const uint64_t m = __ballot(ok);
          if (ok) {
            const uint32_t key = float_key(hv);
            const int p = cnt[j] + lanes_below(m);
            cs[p] = hv;
            ci[p] = s;
            klo[j] = min(klo[j], key);
            khi[j] = max(khi[j], key);
          }
          cnt[j] += __popcll(m);
        }
      };
      static_assert(kSub % 2 == 0, "subtiles go in pairs");
      if (held_s0 + kTStageKeys <= row_n[j]) append(std::true_type{});
      else append(std::false_type{});
    }
  };

  if (tid < 8) sh.want[tid >> 2][tid & 3] = 0;
  for (int i = 0; i < kTBufs - 1 && i < nst; ++i) stage(i);
  wait_stages(min(kTBufs - 2, nst - 1));
  lds_barrier();

  for (int si = 0; si < nst; ++si) {
    const int buf = si % kTBufs;
    if (si > 0) emit_held((si - 1) & 1);
    if (si + kTBufs - 1 < nst) stage(si + kTBufs - 1);
    const int s_stage = si * kTStageKeys;
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) {
      const int sk0 = s_stage + 32 * sub;
      bool any = false;
#pragma unroll
      for (int j = 0; j < QW; ++j) any |= sk0 < row_n[j];
#pragma unroll
      for (int j = 0; j < QW; ++j) held[j][sub] = 0.f;
      if (!any) continue;  // uniform over the wave
      float sc[QW];
      score_subtile<MT, QW>(sh.keys[buf], sh.ksc[buf], 32 * sub + col, half, a, wr, row_scale, sc);
#pragma unroll
      for (int j = 0; j < QW; ++j) held[j][sub] = sc[j];
    }
    held_s0 = s_stage;
    // this wave's flag for the next stage's appends (stage si's keys, then
    // stage si+1's): read after the barrier, rewritten two stages later
    bool near = false;
#pragma unroll
    for (int j = 0; j < QW; ++j) near |= cnt[j] + 2 * kTStageKeys > cap;
    if (lane == 0) sh.want[si & 1][wave] = near;
    wait_stages(min(si + kTBufs - 1, nst - 1) - (si + 1));
    lds_barrier();
  }
  emit_held(nst > 0 ? (nst - 1) & 1 : 0);
#pragma unroll
  for (int j = 0; j < QW; ++j)
    if (row_n[j] > 0) select(j, true);
}

// --------------------------------------------------------------------------
// launchers
// --------------------------------------------------------------------------
hipError_t launch_indexer_f32(const BatchDev &bt, const KeysDev &kd, int num_queries,
                              int max_k_len, int h_i, int d_i, const float *q, const float *w,
                              const float *k, float scale, float *scores, int64_t ld,
                              hipStream_t stream) {
  dim3 grid((max_k_len + kIdxF32Threads - 1) / kIdxF32Threads, num_queries);
  hipLaunchKernelGGL(indexer_f32_kernel, grid, dim3(kIdxF32Threads), 0, stream, bt, kd, h_i, d_i,
                     q, w, k, scale, scores, ld);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// FP8 E4M3 decode form: few query rows over long key ranges.  128-key stages
// (16 KB) arrive by 16-byte global->LDS loads in which 64 consecutive lanes
// cover 1 KB of consecutive key bytes, three stages deep, and their fp32
// scales by 4-byte global->LDS loads.  Each wave scores one
// 32-key tile of every stage.  The 16-byte chunks of a 128-byte key row are
// XOR-permuted (kswz), which spreads the 32 rows a read instruction touches
// over the LDS banks.  The workgroup's page bases are resolved into LDS before
// the loop, so the loop issues no dependent global loads.
// --------------------------------------------------------------------------
constexpr int kDecStageKeys = 128;                 // 4 tiles of 32 keys: one per wave
constexpr int kDecStageBytes = kDecStageKeys * 128;   // 16 KB
constexpr int kDecStageLoads = kDecStageBytes / 1024; // 16 wave-wide key loads per stage
constexpr int kDecStageBufs = 3;
// Keys per workgroup: 1024 (8 stages), or 2048 when the whole grid then fits
// in one round of resident workgroups (three per CU, bounded by LDS; two at
// 128 heads, bounded by registers), which removes the partly filled last
// round (32 x 32k decode: 35.9 -> 33.7 us).  Many blocks of mixed row
// lengths balance better at 1024.
constexpr int staged_resident(int h_i) { return (h_i == 128 ? 2 : 3) * 256; }

template <int KPB>
struct IdxStagedLds {
  uint8_t keys[kDecStageBufs][kDecStageBytes];
  float ksc[kDecStageBufs][kDecStageKeys];
  int64_t page_row[KPB / kPageSize];  // flat row of key 64p of the block (contiguous: s_begin + 64p)
};

template <int MT, int KPB, bool PAGED>
__global__ __launch_bounds__(kIdxThreads) void indexer_fp8_staged_kernel(
    BatchDev bt, KeysDev kd, const uint8_t *__restrict__ q, const float *__restrict__ q_scale,
    const float *__restrict__ w, const uint8_t *__restrict__ k,
    const float *__restrict__ k_scale, float scale, float *__restrict__ scores, int64_t ld) {
  constexpr int H = 32 * MT;
  constexpr int kStagedPages = KPB / kPageSize;
  static_assert(kStagedPages <= kIdxThreads, "one thread per page base");
  __shared__ IdxStagedLds<KPB> sh;
  const int t = blockIdx.y;
  const int b = seq_of_row_wave(bt, t);
  const int n = __builtin_amdgcn_readfirstlane(candidates_of_row(bt, b, t));
  const int s_begin = blockIdx.x * KPB;
  if (s_begin >= n) return;
  const int s_end = min(n, s_begin + KPB);
  const int nst = (s_end - s_begin + kDecStageKeys - 1) / kDecStageKeys;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int half = lane >> 5;
  const int col = lane & 31;

  // query operand: head 32*mt + col, bytes [64*ks + 32*half, +32)
  v8i a[MT][2];
  const uint8_t *qt = q + (int64_t)t * H * 128;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      a[mt][ks] = *(const v8i *)(qt + (32 * mt + col) * 128 + 64 * ks + 32 * half);
  // head weights of the accumulator rows this lane holds (rows 8r + 4*half + 0..3)
  float wr[MT][16];
  const float *wt = w + (int64_t)t * H;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const float4 v = *(const float4 *)(wt + 32 * mt + 8 * r4 + 4 * half);
      wr[mt][4 * r4 + 0] = v.x;
      wr[mt][4 * r4 + 1] = v.y;
      wr[mt][4 * r4 + 2] = v.z;
      wr[mt][4 * r4 + 3] = v.w;
    }
  const float row_scale = q_scale[t] * scale;
  float *out = scores + (int64_t)t * ld;
  // page bases of the block (paged layout; a contiguous one addresses rows directly)
  if (PAGED && threadIdx.x < kStagedPages) {
    const int s = min(s_begin + kPageSize * (int)threadIdx.x, n - 1);
    sh.page_row[threadIdx.x] = key_row(kd, b, s & ~(kPageSize - 1));
  }
  const int64_t kbase = PAGED ? 0 : kd.k_seq_start[b];
  auto row_of = [&](int s) __attribute__((always_inline)) -> int64_t {
    if constexpr (PAGED) return sh.page_row[(s - s_begin) >> kPageShift] + (s & (kPageSize - 1));
    else return kbase + s;
  };
  // The query, weight and page loads must be complete (and known complete
  // to the compiler) before the stage loads are issued: otherwise its wait
  // bookkeeping would later wait for them behind stage loads kept in flight.
  // (The barrier alone does not wait for global loads.)
  wait_vmcnt<0>();
  __syncthreads();

  const uint32_t keys0 = __builtin_amdgcn_readfirstlane(lds_addr(&sh.keys[0][0]));
  const uint32_t ksc0 = __builtin_amdgcn_readfirstlane(lds_addr(&sh.ksc[0][0]));
  // stage si -> buffer si % 3.  Key load j (wave + 4m) covers keys 8j .. 8j+7
  // of the stage: lane i stores chunk i % 8 of key 8j + i/8, which holds the
  // key's chunk (i % 8) ^ kswz(key).  Waves 0 and 1 also load the scales of
  // keys 64*wave .. +63.  Keys past n reload key n - 1.
  auto stage = [&](int si) __attribute__((always_inline)) {
    const int buf = si % kDecStageBufs;
    const int s_stage = s_begin + si * kDecStageKeys;
#pragma unroll
    for (int m = 0; m < kDecStageLoads / 4; ++m) {
      const int j = wave + 4 * m;
      const int r = 8 * j + (lane >> 3);
      const int s = min(s_stage + r, n - 1);
      const int64_t row = row_of(s);
      lds_dma16_at(k + row * 128 + 16 * ((lane & 7) ^ kswz(r)), keys0 + buf * kDecStageBytes + 1024 * j);
    }
    if (wave < 2) {
      const int s = min(s_stage + 64 * wave + lane, n - 1);
      const int64_t row = row_of(s);
      lds_dma4_at(k_scale + row, ksc0 + buf * (kDecStageKeys * 4) + 256 * wave);
    }
  };
  constexpr int kLoads = kDecStageLoads / 4;  // key loads per wave per stage (+1 for waves 0, 1)
  // wait until at most `o` of this wave's most recent stages may be in flight
  auto wait_stages = [&](int o) __attribute__((always_inline)) {
    if (wave < 2) {
      if (o >= 2) wait_vmcnt<2 * (kLoads + 1)>(); else if (o == 1) wait_vmcnt<kLoads + 1>(); else wait_vmcnt<0>();
    } else {
      if (o >= 2) wait_vmcnt<2 * kLoads>(); else if (o == 1) wait_vmcnt<kLoads>(); else wait_vmcnt<0>();
    }
  };
  static_assert(kDecStageBufs <= 4, "at most three stages in flight");

  // stages 0 .. B-2 in flight, then wait for stage 0
  for (int i = 0; i < kDecStageBufs - 1 && i < nst; ++i) stage(i);
  wait_stages(min(kDecStageBufs - 2, nst - 1));
  lds_barrier();

  // B operand reads: key r = 32*wave + col of the stage, chunks 4ks + 2half, +1
  const int r = 32 * wave + col;
  for (int si = 0; si < nst; ++si) {
    const int buf = si % kDecStageBufs;
    if (si + kDecStageBufs - 1 < nst) stage(si + kDecStageBufs - 1);
    const uint8_t *kb = sh.keys[buf] + r * 128;
    float sum = 0.f;
    v8i bk[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = 4 * ks + 2 * half;
      const v4i lo = *(const v4i *)(kb + 16 * (c ^ kswz(r)));
      const v4i up = *(const v4i *)(kb + 16 * ((c + 1) ^ kswz(r)));
      bk[ks] = v8i{lo.x, lo.y, lo.z, lo.w, up.x, up.y, up.z, up.w};
    }
    const float ksc = sh.ksc[buf][r];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      v16f acc = {};
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[mt][0], bk[0], acc, 0, 0, 0, 127, 0, 127);
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[mt][1], bk[1], acc, 0, 0, 0, 127, 0, 127);
#pragma unroll
      for (int i = 0; i < 16; ++i) sum = fmaf(wr[mt][i], relu(acc[i]), sum);
    }
    sum = add_halves(sum);
    const int s = s_begin + si * kDecStageKeys + r;
    if (half == 0 && s < s_end) out[s] = sum * row_scale * ksc;
    // the next stage must have landed; later ones may stay in flight
    wait_stages(min(si + kDecStageBufs, nst) - (si + 2));
    lds_barrier();
  }
}

// A row's list holds 3k + one stage of candidates.  A compaction reads the
// list in one histogram pass and one ordered rewrite (it keeps the boundary
// bin of the first digit, a lower bound on the k-th key, whenever that frees
// half the list), so compactions are cheap and a short list keeps the final
// selection small.  Measured with these compactions (indexer + top-k):
// prefill_16k 1.64, 1.38, 1.48 ms at lists of 2k, 3k, 4k; prefill_64k 22.0,
// 19.3, 19.2, 19.3, 19.0-19.4, 19.1-19.4 ms at 2k .. 7k (flat from 3k).  The
// history length no longer enters.
int fused_topk_cap(int k, int max_k_len) {
  (void)max_k_len;
  return (int)(((int64_t)3 * k + kTStageKeys + 63) / 64 * 64);
}

size_t fused_topk_workspace_bytes(int num_queries, int k, int max_k_len) {
  // candidate scores, then candidate positions (each 256-byte aligned)
  const size_t one = ((size_t)num_queries * fused_topk_cap(k, max_k_len) * 4 + 255) / 256 * 256;
  return 2 * one;
}

hipError_t launch_indexer_topk_fused(const BatchDev &bt, const KeysDev &kd, int num_seqs, int num_queries,
                                     int max_q_per_seq, int max_k_len, int h_i, const uint8_t *q,
                                     const float *q_scale, const float *w, const uint8_t *k, const float *k_scale,
                                     float scale, int topk, int32_t *indices, void *workspace, hipStream_t stream) {
  if (num_queries == 0) return hipSuccess;
  if (kd.paged && max_k_len > kFusedMaxPages * kPageSize) return hipErrorInvalidValue;
  const int cap = fused_topk_cap(topk, max_k_len);
  const size_t one = ((size_t)num_queries * cap * 4 + 255) / 256 * 256;
  float *cand_s = (float *)workspace;
  int32_t *cand_i = (int32_t *)((char *)workspace + one);
  // two rows a wave, one at 128 heads (whose query block and weights fill the registers)
  const int qw = h_i == 128 ? 1 : 2;
  const dim3 grid((max_q_per_seq + 4 * qw - 1) / (4 * qw), num_seqs);
#define DSA_FUSED(MT, QW)                                                                                       \
  do {                                                                                                          \
    if (kd.paged)                                                                                               \
      hipLaunchKernelGGL((indexer_topk_fused_kernel<MT, QW, true>), grid, dim3(kIdxThreads), 0, stream, bt, kd, \
                         q, q_scale, w, k, k_scale, scale, topk, cap, cand_s, cand_i, indices);                 \
    else                                                                                                        \
      hipLaunchKernelGGL((indexer_topk_fused_kernel<MT, QW, false>), grid, dim3(kIdxThreads), 0, stream, bt,    \
                         kd, q, q_scale, w, k, k_scale, scale, topk, cap, cand_s, cand_i, indices);             \
  } while (0)
  switch (h_i) {
    case 32: DSA_FUSED(1, 2); break;
    case 64: DSA_FUSED(2, 2); break;
    case 128: DSA_FUSED(4, 1); break;
    default: return hipErrorInvalidValue;
  }
#undef DSA_FUSED
  return hipGetLastError();
}

hipError_t launch_indexer_fp8(const BatchDev &bt, const KeysDev &kd, int num_seqs, int num_queries,
                              int max_q_per_seq, int max_k_len, int h_i, const uint8_t *q,
                              const float *q_scale, const float *w, const uint8_t *k,
                              const float *k_scale, float scale, float *scores, int64_t ld,
                              hipStream_t stream) {
  if (max_q_per_seq >= 8) {
    // two rows a wave, one at 128 heads (whose query block and weights fill the registers)
    const int qw = h_i == 128 ? 1 : 2;
    const dim3 grid((max_k_len + kTKeysPerBlock - 1) / kTKeysPerBlock, (max_q_per_seq + 4 * qw - 1) / (4 * qw),
                    num_seqs);
#define DSA_TILED(MT, QW)                                                                                       \
  do {                                                                                                             \
    if (kd.paged)                                                                                                  \
      hipLaunchKernelGGL((indexer_fp8_tiled_kernel<MT, QW, true>), grid, dim3(kIdxThreads), 0, stream, bt, kd, q, \
                         q_scale, w, k, k_scale, scale, scores, ld);                                               \
    else                                                                                                           \
      hipLaunchKernelGGL((indexer_fp8_tiled_kernel<MT, QW, false>), grid, dim3(kIdxThreads), 0, stream, bt, kd,   \
                         q, q_scale, w, k, k_scale, scale, scores, ld);                                            \
  } while (0)
    switch (h_i) {
      case 32: DSA_TILED(1, 2); break;
      case 64: DSA_TILED(2, 2); break;
      case 128: DSA_TILED(4, 1); break;
      default: return hipErrorInvalidValue;
    }
#undef DSA_TILED
    return hipGetLastError();
  }
  const bool one_round = (int64_t)((max_k_len + 2047) / 2048) * num_queries <= staged_resident(h_i);
  const int kpb = one_round ? 2048 : 1024;
  dim3 grid((max_k_len + kpb - 1) / kpb, num_queries);
#define DSA_STAGED(MT, KPB)                                                                                       \
  do {                                                                                                            \
    if (kd.paged)                                                                                                 \
      hipLaunchKernelGGL((indexer_fp8_staged_kernel<MT, KPB, true>), grid, dim3(kIdxThreads), 0, stream, bt, kd, \
                         q, q_scale, w, k, k_scale, scale, scores, ld);                                           \
    else                                                                                                          \
      hipLaunchKernelGGL((indexer_fp8_staged_kernel<MT, KPB, false>), grid, dim3(kIdxThreads), 0, stream, bt,    \
                         kd, q, q_scale, w, k, k_scale, scale, scores, ld);                                       \
  } while (0)
  switch (h_i) {
    case 32:
      if (one_round) DSA_STAGED(1, 2048); else DSA_STAGED(1, 1024);
      break;
    case 64:
      if (one_round) DSA_STAGED(2, 2048); else DSA_STAGED(2, 1024);
      break;
    case 128:
      if (one_round) DSA_STAGED(4, 2048); else DSA_STAGED(4, 1024);
      break;
    default:
      return hipErrorInvalidValue;
  }
#undef DSA_STAGED
  return hipGetLastError();
}

}  // namespace dsa
