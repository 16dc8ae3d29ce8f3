// Per-row causal top-k (gfx950).
//
// For query row t with n_t candidates, writes the positions of the
// m = min(k, n_t) largest scores in ascending order, then -1 padding
// ("DeepSeek Sparse Attention DSA Architecture Guide", "Stage 2: Fine-Grained
// Token Selection", TopK equation; its implementation section keeps
// k = min(top_k, seq_len) and re-sorts the chosen positions into temporal
// order).  Ties go to the lowest position, so the result is unique and the
// kernel is deterministic.
//
// One 1024-thread workgroup owns a row and keeps its first 32768 scores (the
// whole row when it fits) in LDS.  Selection is exact:
//   1. min / max of the row (while caching it);
//   2. histogram of a monotone linear binning of the values into 2048 bins
//      (spreads typical score distributions evenly, so LDS atomics rarely
//      collide); a wave-wide scan from the top finds the bin b* holding the
//      k-th largest score;
//   3. the elements of bin b* only -- compacted into an LDS list when there
//      are at most 1024 of them -- give the threshold key tau and how many
//      elements equal to tau are kept: by direct ranking (key descending,
//      position ascending) when the list holds at most 256, else by an exact
//      radix select (11/11/10-bit digits of an order-preserving uint32 key);
//   4. one ordered pass writes key > tau, plus the first `need_eq` elements
//      equal to tau, at positions given by block scans of per-thread (row in
//      LDS) or per-wave (longer rows) counts: the output comes out ascending.
#include <algorithm>

#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkCache = 32768;  // scores kept in LDS (128 KiB)
constexpr int kTkBins = 2048;
constexpr int kTkCand = 1024;
constexpr int kTkRankMax = 256;  // bins up to this size are resolved by direct ranking

struct TopkLds {
  float cache[kTkCache];
  uint32_t hist[kTkBins];
  int32_t cand[kTkCand];
  uint32_t cand_key[kTkCand];
  uint32_t red_lo[kTkWaves];
  uint32_t red_hi[kTkWaves];
  int32_t cnt[2][2][kTkWaves];
  int32_t scan_bin;
  int32_t scan_above;
  int32_t cand_count;
  uint32_t rank_tau;
  int32_t rank_need_eq;
};

__device__ __forceinline__ float key_to_float(uint32_t key) {
  uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  for (int off = 32; off > 0; off >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Wave 0 only.  Finds the bin d such that the count strictly above d is
// < need and the count from d upward is >= need.  Two wave-wide scans: lane l
// first sums the l-th group of nbins/64 bins counted from the top and an
// inclusive lane scan picks the group; then the group's bins, one per lane,
// are scanned the same way.
__device__ void scan_from_top(const uint32_t *hist, int nbins, int need, int32_t *out_bin,
                              int32_t *out_above) {
  const int lane = lane_id();
  const int c = nbins / 64;
  const int hi = nbins - lane * c;
  int s = 0;
  // lane l reads its group in the rotated order (j + l) % c, so that at every
  // step the wave's 64 reads fall into distinct LDS banks
  for (int j = 0; j < c; ++j) s += (int)hist[hi - 1 - ((j + lane) & (c - 1))];
  int incl = s;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  const uint64_t hit = __ballot(incl >= need);
  if (hit == 0) {  // only with NaN scores (a precondition violation)
    if (lane == 0) { *out_bin = 0; *out_above = 0; }
    return;
  }
  const int grp = __ffsll((unsigned long long)hit) - 1;
  const int above_grp = __shfl(incl - s, grp, 64);
  const int top = nbins - grp * c;  // one past the group's highest bin
  const int v = lane < c ? (int)hist[top - 1 - lane] : 0;
  int incl2 = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl2, off, 64);
    if (lane >= off) incl2 += y;
  }
  const uint64_t hit2 = __ballot(lane < c && above_grp + incl2 >= need);
  const int j = hit2 ? __ffsll((unsigned long long)hit2) - 1 : c - 1;  // empty only with NaN scores
  const int above = above_grp + __shfl(incl2 - v, j, 64);
  if (lane == 0) {
    *out_bin = top - 1 - j;
    *out_above = above;
  }
}

// Loads of one sweep chunk: kU float4 per thread, all issued before any is
// used (a plain loop would wait out one memory latency per load).
constexpr int kU = 8;
constexpr int kChunk = 4 * kU * kTkThreads;  // elements per sweep chunk (32768)

__device__ __forceinline__ void load_chunk(const float *src, int base, int n, float4 (&v)[kU]) {
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int i = base + 4 * ((int)threadIdx.x + u * kTkThreads);
    v[u] = i < n ? *(const float4 *)(src + i) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// Long rows in small batches are selected in two passes (launch_topk).  A
// row's candidate list holds, part after part, the winners of each
// kTkCache-long part of the row: min(k, part length) positions, ascending,
// and their scores.  Part pass: workgroup (t, p) selects from its part and
// writes its winners at the part's offset in the list.  Merge pass: the row's
// list is the input row, and the positions its winners stand for are written.
// Every element of the row's top-k has fewer than k elements ahead of it, in
// its part too, so it is among its part's winners; list order is position
// order, so ties still go to the lowest position.
struct TopkSplit {
  int32_t parts;    // 0: one pass
  int32_t merge;    // 0: part pass, 1: merge pass
  int32_t *cpos;    // [T, ld_c] candidate positions
  float *cval;      // [T, ld_c] candidate scores
  int64_t ld_c;     // list stride: >= the longest list, a multiple of 4
  int32_t lim;      // max_k_len: reads of a score row stay below it (ld >= max_k_len)
};

// Length of row t's candidate list up to (not including) part p.
__device__ __forceinline__ int list_offset(int n_row, int k, int p) {
  int off = 0;
  for (int q = 0; q < p; ++q) off += min(k, min(max(n_row - q * kTkCache, 0), kTkCache));
  return off;
}

template <bool EARLY>
__global__ __launch_bounds__(kTkThreads) void topk_kernel(BatchDev bt,
                                                         const float *__restrict__ scores,
                                                         int64_t ld, int k,
                                                         int32_t *__restrict__ indices,
                                                         TopkSplit sp) {
  __shared__ TopkLds sh;
  const int t = blockIdx.x;
  // EARLY (decode rows: one query row per sequence, selected in one pass):
  // the row's first sweep chunk is loaded before its length is known, so
  // that the length lookup's memory round trip passes under it.  The loads
  // stop at max_k_len, inside the row, and elements past the row's
  // candidates are never used (every use below tests i < n).  Causal
  // prefill rows and the parts of long rows are often far shorter than
  // max_k_len: there such loads would read mostly unused scores, so the
  // launcher takes the other instantiation.
  float4 v0[kU];
  if constexpr (EARLY) load_chunk(scores + (int64_t)t * ld, 0, min(sp.lim, kTkCache), v0);
  const int b = seq_of_row_wave(bt, t);
  const int n_row = candidates_of_row(bt, b, t);
  int n = n_row;
  const float *row = scores + (int64_t)t * ld;
  int32_t *out = indices + (int64_t)t * k;
  int pos_off = 0;                   // part pass: first position of the part
  const int32_t *pos_map = nullptr;  // merge pass: the positions list entries stand for
  float *val_out = nullptr;          // part pass: scores of the winners
  if (sp.parts > 0 && !sp.merge) {
    const int p = blockIdx.y;
    pos_off = p * kTkCache;
    n = min(max(n_row - pos_off, 0), kTkCache);
    row += pos_off;
    const int64_t off = (int64_t)t * sp.ld_c + list_offset(n_row, k, p);
    out = sp.cpos + off;
    val_out = sp.cval + off;
  } else if (sp.parts > 0) {
    n = list_offset(n_row, k, sp.parts);
    row = sp.cval + (int64_t)t * sp.ld_c;
    pos_map = sp.cpos + (int64_t)t * sp.ld_c;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  if (n <= k) {  // every candidate is kept
    if (val_out) {  // part pass: the whole part, no padding (the next part's entries follow)
      for (int i = tid; i < n; i += kTkThreads) {
        out[i] = pos_off + i;
        val_out[i] = row[i];
      }
    } else {
      for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? (pos_map ? pos_map[i] : i) : -1;
    }
    return;
  }
  // The first sweep keeps the row's first chunk (all of it when n <= 32768)
  // in LDS; every later sweep reads that chunk from there.
  static_assert(kChunk == kTkCache, "the cached part of a row is its first sweep chunk");
  const bool cached = n <= kTkCache;
#define DSA_SWEEP_CHUNK(base, v)                   \
  if (base == 0) load_chunk(sh.cache, base, n, v); \
  else load_chunk(row, base, n, v);

  // ---- 1. cache the row, min / max key ----
  // (min / max on the values; the keys of the two extremes are taken once,
  // which folds -0 onto +0 as the keys of every element would)
  float vmin = INFINITY, vmax = -INFINITY;
  for (int base = 0; base < n; base += kChunk) {
    float4 v[kU];
    if (EARLY && base == 0) {
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = v0[u];
    } else {
      load_chunk(row, base, n, v);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + 4 * (tid + u * kTkThreads);
      if (base == 0 && i < n) *(float4 *)(&sh.cache[i]) = v[u];
      if (i + 3 < n) {
        vmin = fminf(vmin, fminf(fminf(v[u].x, v[u].y), fminf(v[u].z, v[u].w)));
        vmax = fmaxf(vmax, fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w)));
      } else {
        const float f[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (i + j < n) {
            vmin = fminf(vmin, f[j]);
            vmax = fmaxf(vmax, f[j]);
          }
      }
    }
  }
  uint32_t kmin = wave_min_u32(float_key(vmin));
  uint32_t kmax = wave_max_u32(float_key(vmax));
  if (lane == 0) { sh.red_lo[wave] = kmin; sh.red_hi[wave] = kmax; }
  for (int i = tid; i < kTkBins; i += kTkThreads) sh.hist[i] = 0;
  lds_barrier();
  kmin = sh.red_lo[0];
  kmax = sh.red_hi[0];
  for (int w2 = 1; w2 < kTkWaves; ++w2) {
    kmin = min(kmin, sh.red_lo[w2]);
    kmax = max(kmax, sh.red_hi[w2]);
  }
  const float fmin = key_to_float(kmin);
  const float fmax = key_to_float(kmax);
  float inv = (float)kTkBins / (fmax - fmin);
  if (!(fmax > fmin) || !(inv < 3.0e38f)) inv = 0.f;  // degenerate range: one bin
  // (a NaN score, a precondition violation, converts to bin 0)
  auto bin_of = [&](float f) -> int {
    return (int)__builtin_amdgcn_fmed3f((f - fmin) * inv, 0.f, (float)(kTkBins - 1));
  };

  // ---- 2. histogram, threshold bin ----
  // The lowest bin takes the row minimum with all its duplicates (the exact
  // zeros of ReLU scores): each thread counts those in a register and adds
  // them once, instead of every thread hitting one LDS counter per element.
  uint32_t low = 0u;
  for (int base = 0; base < n; base += kChunk) {
    float4 v[kU];
    DSA_SWEEP_CHUNK(base, v);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + 4 * (tid + u * kTkThreads);
      const float f[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      const bool whole = i + 3 < n;  // no per-element bound test inside the row
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (whole || i + j < n) {
          const int bn = bin_of(f[j]);
          if (bn == 0)
            ++low;
          else
            atomicAdd(&sh.hist[bn], 1u);
        }
      }
    }
  }
  if (low) atomicAdd(&sh.hist[0], low);
  lds_barrier();
  if (wave == 0) scan_from_top(sh.hist, kTkBins, k, &sh.scan_bin, &sh.scan_above);
  lds_barrier();
  const int bstar = sh.scan_bin;
  int need = k - sh.scan_above;
  const int bcount = (int)sh.hist[bstar];
  const bool use_list = bcount <= kTkCand;
  if (tid == 0) sh.cand_count = 0;
  lds_barrier();

  // A cached row (n <= 32768) is one piece: thread tid owns the contiguous
  // run [tid*R, tid*R + R), R <= 32 a multiple of 4.  Rotated read order:
  // when R divides 64, 64/R runs share a 256-byte row of the 64 LDS banks
  // and run tid starts at tid*R/64, so 16 neighbouring lanes read 16
  // different 16-byte bank groups (a rotation by tid alone maps lanes l and
  // l+8, at R = 32, or all 16 lanes, at R = 16, to one group).  Other run
  // lengths rotate by tid.
  const int R = ((min(n, kChunk) + kTkThreads - 1) / kTkThreads + 3) & ~3;
  const int r0 = tid * R;
  const int r4 = R / 4;
  const int rot = (64 % R == 0 ? (tid * R) >> 6 : tid) % r4;
  // When the row is cached and bin b* fits the candidate list, the list is
  // built from the runs, and each thread keeps bitmasks of its elements in
  // bins above b* (all above tau: the binning is monotone) and in b*; the
  // ordered pass then re-tests only the in-bin elements against tau.
  const bool run_masks = cached && use_list;
  uint32_t above_bin = 0u, in_bin = 0u;

  // ---- 3. exact threshold inside bin b* ----
  if (run_masks) {
    for (int q = 0; q < r4; ++q) {
      const int qq = q + rot < r4 ? q + rot : q + rot - r4;
      const int i = r0 + 4 * qq;
      if (i >= n) continue;
      const float4 v = *(const float4 *)(&sh.cache[i]);
      const float f[4] = {v.x, v.y, v.z, v.w};
      const bool whole = i + 3 < n;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!whole && i + j >= n) break;
        const int bn = bin_of(f[j]);
        above_bin |= (uint32_t)(bn > bstar) << (4 * qq + j);
        if (bn == bstar) {
          in_bin |= 1u << (4 * qq + j);
          const int slot = atomicAdd(&sh.cand_count, 1);
          if (slot < kTkCand) {
            sh.cand[slot] = i + j;
            sh.cand_key[slot] = float_key(f[j]);
          }
        }
      }
    }
    lds_barrier();
  } else if (use_list) {
    for (int base = 0; base < n; base += kChunk) {
      float4 v[kU];
      DSA_SWEEP_CHUNK(base, v);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = base + 4 * (tid + u * kTkThreads);
        const float f[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (i + j < n && bin_of(f[j]) == bstar) {
            const int slot = atomicAdd(&sh.cand_count, 1);
            if (slot < kTkCand) {
              sh.cand[slot] = i + j;
              sh.cand_key[slot] = float_key(f[j]);
            }
          }
      }
    }
    lds_barrier();
  }
  const int ncand = min(bcount, kTkCand);
  uint32_t prefix = 0u, pmask = 0u;
  const bool by_rank = use_list && ncand <= kTkRankMax;
  if (by_rank) {
    // Candidate c ranks by (key descending, position ascending); the one at
    // rank need-1 is the last kept: its key is tau, and need_eq is what is
    // left of `need` after the candidates strictly above tau.
    if (tid < ncand) {
      const uint32_t ki = sh.cand_key[tid];
      const int pi = sh.cand[tid];
      int rank = 0, gt = 0;
      for (int j = 0; j < ncand; ++j) {
        const uint32_t kj = sh.cand_key[j];
        const int pj = sh.cand[j];
        gt += kj > ki;
        rank += (kj > ki) | ((kj == ki) & (pj < pi));
      }
      if (rank == need - 1) {
        sh.rank_tau = ki;
        sh.rank_need_eq = need - gt;
      }
    }
    lds_barrier();
    prefix = sh.rank_tau;
    need = sh.rank_need_eq;
  }
#pragma unroll 1
  for (int pass = 0; pass < (by_rank ? 0 : 3); ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int i = tid; i < nb; i += kTkThreads) sh.hist[i] = 0;
    lds_barrier();
    if (use_list) {
      for (int c = tid; c < ncand; c += kTkThreads) {
        const int pos = sh.cand[c];
        const uint32_t key = float_key(pos < kTkCache ? sh.cache[pos] : row[pos]);
        if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & (nb - 1)], 1u);
      }
    } else {
      for (int base = 0; base < n; base += kChunk) {
        float4 v[kU];
        DSA_SWEEP_CHUNK(base, v);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i = base + 4 * (tid + u * kTkThreads);
          const float f[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t key = float_key(f[j]);
            if (i + j < n && bin_of(f[j]) == bstar && (key & pmask) == prefix)
              atomicAdd(&sh.hist[(key >> shift) & (nb - 1)], 1u);
          }
        }
      }
    }
    lds_barrier();
    if (wave == 0) scan_from_top(sh.hist, nb, need, &sh.scan_bin, &sh.scan_above);
    lds_barrier();
    need -= sh.scan_above;
    prefix |= (uint32_t)sh.scan_bin << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    lds_barrier();
  }
  const uint32_t tau = prefix;
  const int need_eq = need;

  // ---- 4. ordered write: key > tau, then the first need_eq keys == tau ----
  // (a part pass always holds its part in LDS: parts are kTkCache long)
  auto emit = [&](int pos, int pos_i) __attribute__((always_inline)) {
    out[pos] = pos_map ? pos_map[pos_i] : pos_off + pos_i;
    if (val_out) val_out[pos] = sh.cache[pos_i];
  };
  int gt_run = 0, eq_run = 0;
  if (cached) {
    // The row is in LDS, one piece of runs (above).  Each thread holds
    // bitmasks of its run's elements above and equal to tau; one block-wide
    // exclusive scan of the two counts gives every run its output offset, so
    // the output comes out ascending without any per-element synchronisation.
    {
      uint32_t gtm = 0u, eqm = 0u;
      if (run_masks) {
        gtm = above_bin;
        for (uint32_t m = in_bin; m; m &= m - 1) {
          const int bit = __ffs(m) - 1;
          const uint32_t key = float_key(sh.cache[r0 + bit]);
          gtm |= (uint32_t)(key > tau) << bit;
          eqm |= (uint32_t)(key == tau) << bit;
        }
      } else {
        for (int q = 0; q < r4; ++q) {
          const int qq = q + rot < r4 ? q + rot : q + rot - r4;
          const int i = r0 + 4 * qq;
          if (i >= n) continue;
          const float4 v = *(const float4 *)(&sh.cache[i]);
          const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (i + j >= n) break;
            const uint32_t key = float_key(f[j]);
            gtm |= (uint32_t)(key > tau) << (4 * qq + j);
            eqm |= (uint32_t)(key == tau) << (4 * qq + j);
          }
        }
      }
      const int gc = __popc(gtm), ec = __popc(eqm);
      // block-wide exclusive scan of (gc, ec) <= 32: lanes by bit-plane
      // ballots (six planes each), then waves through LDS
      int gi = 0, ei = 0, gwave = 0, ewave = 0;
#pragma unroll
      for (int bit = 0; bit < 6; ++bit) {
        const uint64_t bg = __ballot((gc >> bit) & 1), be = __ballot((ec >> bit) & 1);
        gi += lanes_below(bg) << bit;
        ei += lanes_below(be) << bit;
        gwave += __popcll(bg) << bit;
        ewave += __popcll(be) << bit;
      }
      if (lane == 0) { sh.cnt[0][0][wave] = gwave; sh.cnt[0][1][wave] = ewave; }
      lds_barrier();
      int gw = 0, ew = 0, gb = 0, eb = 0;
      for (int w2 = 0; w2 < kTkWaves; ++w2) {
        const int gv = sh.cnt[0][0][w2], ev = sh.cnt[0][1][w2];
        if (w2 < wave) { gw += gv; ew += ev; }
        gb += gv;
        eb += ev;
      }
      int g_before = gt_run + gw + gi;
      int e_before = eq_run + ew + ei;
      uint32_t m = gtm | eqm;
      while (m) {
        const int bit = __ffs(m) - 1;
        m &= m - 1;
        const int pos_i = r0 + bit;
        if ((gtm >> bit) & 1u) {
          const int pos = g_before + min(e_before, need_eq);
          if (pos < k) emit(pos, pos_i);
          ++g_before;
        } else {
          if (e_before < need_eq) {
            const int pos = g_before + e_before;
            if (pos < k) emit(pos, pos_i);
          }
          ++e_before;
        }
      }
      gt_run += gb;
      eq_run += eb;
    }
  } else {
    // The row is read in pieces of 32768 elements (the first from LDS), each
    // cut into one 2048-element segment per wave; lane l holds elements
    // 256*u + 4*l + j (u < 8, j < 4) of its wave's segment, so every wave-wide
    // load is one contiguous 1 KB and all eight are in flight together.  The
    // waves' counts above and equal to tau, exchanged once through LDS, give
    // each wave its output offsets; inside a wave, ballots of the per-lane
    // counts give each lane its offsets, run by run.
    constexpr int kSeg = kChunk / kTkWaves;  // 2048
    int par = 0;
    for (int p0 = 0; p0 < n; p0 += kChunk, par ^= 1) {
      const int s0 = p0 + wave * kSeg + 4 * lane;
      float4 v[kU];
      if (p0 == 0) {  // the cached first piece
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i = s0 + 256 * u;
          v[u] = i < n ? *(const float4 *)(&sh.cache[i]) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      } else {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i = s0 + 256 * u;
          v[u] = i < n ? *(const float4 *)(row + i) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      uint32_t gtm = 0u, eqm = 0u;  // bit 4u+j: element s0 + 256u + j
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float f[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool in = s0 + 256 * u + j < n;
          const uint32_t key = float_key(f[j]);
          gtm |= (uint32_t)(in && key > tau) << (4 * u + j);
          eqm |= (uint32_t)(in && key == tau) << (4 * u + j);
        }
      }
      int gw = __popc(gtm), ew = __popc(eqm);
      for (int off = 32; off > 0; off >>= 1) {
        gw += __shfl_xor(gw, off, 64);
        ew += __shfl_xor(ew, off, 64);
      }
      // the counts are double-buffered over pieces: the barrier of the next
      // piece separates these reads from the next writes of the same buffer
      if (lane == 0) { sh.cnt[par][0][wave] = gw; sh.cnt[par][1][wave] = ew; }
      lds_barrier();
      int g_before = gt_run, e_before = eq_run, gb = 0, eb = 0;
      for (int w2 = 0; w2 < kTkWaves; ++w2) {
        const int gv = sh.cnt[par][0][w2], ev = sh.cnt[par][1][w2];
        if (w2 < wave) { g_before += gv; e_before += ev; }
        gb += gv;
        eb += ev;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t gn = (gtm >> (4 * u)) & 15u, en = (eqm >> (4 * u)) & 15u;
        const int cg = __popc(gn), ce = __popc(en);
        // exclusive lane prefix and wave total of cg, ce (0..4: three bit planes)
        int pg = 0, pe = 0, tg = 0, te = 0;
#pragma unroll
        for (int bit = 0; bit < 3; ++bit) {
          const uint64_t bg = __ballot((cg >> bit) & 1), be = __ballot((ce >> bit) & 1);
          pg += lanes_below(bg) << bit;
          pe += lanes_below(be) << bit;
          tg += __popcll(bg) << bit;
          te += __popcll(be) << bit;
        }
        int gpos = g_before + pg, epos = e_before + pe;
        uint32_t m = gn | en;
        while (m) {
          const int j = __ffs(m) - 1;
          m &= m - 1;
          const int pos_i = s0 + 256 * u + j;
          if ((gn >> j) & 1u) {
            const int pos = gpos + min(epos, need_eq);
            if (pos < k) emit(pos, pos_i);
            ++gpos;
          } else {
            if (epos < need_eq) {
              const int pos = gpos + epos;
              if (pos < k) emit(pos, pos_i);
            }
            ++epos;
          }
        }
        g_before += tg;
        e_before += te;
      }
      gt_run += gb;
      eq_run += eb;
    }
  }
  const int total = gt_run + min(eq_run, need_eq);
  if (!val_out)
    for (int i = total + tid; i < k; i += kTkThreads) out[i] = -1;
#undef DSA_SWEEP_CHUNK
}

// Few rows with histories past the LDS row cache leave most CUs idle while
// one workgroup sweeps each long row; such batches take the two passes.
static int topk_parts(int num_queries, int max_k_len) {
  if (num_queries >= 256 || max_k_len <= kTkCache) return 0;
  return (max_k_len + kTkCache - 1) / kTkCache;
}

// List stride: a row's list holds min(k, part length) per part, never more
// than the row itself.
static int64_t topk_list_ld(int parts, int k, int max_k_len) {
  return (std::min((int64_t)parts * k, (int64_t)max_k_len) + 3) / 4 * 4;
}

size_t topk_workspace_bytes(int num_queries, int max_k_len, int k) {
  const int parts = topk_parts(num_queries, max_k_len);
  if (!parts) return 0;
  const size_t list = (size_t)num_queries * topk_list_ld(parts, k, max_k_len) * 4;
  return (list + 255) / 256 * 256 * 2;  // positions, then scores
}

hipError_t launch_topk(const BatchDev &bt, int num_queries, int max_k_len, const float *scores, int64_t ld,
                       int k, int32_t *indices, void *workspace, hipStream_t stream) {
  if (num_queries == 0) return hipSuccess;
  TopkSplit sp{};
  sp.lim = max_k_len;
  sp.parts = topk_parts(num_queries, max_k_len);
  if (!sp.parts) {
    if (bt.one_per_seq)
      hipLaunchKernelGGL(topk_kernel<true>, dim3(num_queries), dim3(kTkThreads), 0, stream, bt, scores, ld, k,
                         indices, sp);
    else
      hipLaunchKernelGGL(topk_kernel<false>, dim3(num_queries), dim3(kTkThreads), 0, stream, bt, scores, ld, k,
                         indices, sp);
    return hipGetLastError();
  }
  sp.ld_c = topk_list_ld(sp.parts, k, max_k_len);
  const size_t list = ((size_t)num_queries * sp.ld_c * 4 + 255) / 256 * 256;
  sp.cpos = (int32_t *)workspace;
  sp.cval = (float *)((char *)workspace + list);
  hipLaunchKernelGGL(topk_kernel<false>, dim3(num_queries, sp.parts), dim3(kTkThreads), 0, stream, bt, scores, ld, k,
                     indices, sp);
  sp.merge = 1;
  hipLaunchKernelGGL(topk_kernel<false>, dim3(num_queries), dim3(kTkThreads), 0, stream, bt, scores, ld, k, indices,
                     sp);
  return hipGetLastError();
}

}  // namespace dsa
