"""Seeded synthetic inputs for the DSA hot path.

This module only draws random numbers, lays them out and stores them in the
input formats (bfloat16 rounding, per-token FP8 E4M3 encoding).  It holds
none of the method's arithmetic: no score, selection or attention is
computed here.  Both the HIP library's tests and the CPU oracle take their
inputs from it, so it must stay free of either side's code.

Determinism: every tensor is drawn in chunks of 256 rows, chunk c of tensor
``tid`` from ``numpy.random.default_rng([seed, tid, *sub, c])``.  Any row
range can therefore be regenerated on its own (the oracle checks sampled
rows of workloads far too large to hold twice).

Tensor ids: 0 context lengths, 1 indexer queries q^I, 2 head weights w,
3 indexer keys k^I, 4 MLA queries q, 5 latent cache rows kv, 6 structure
(needles, block drift), 7 page permutation.

The five workloads are the ones the library is measured on:
  tiny_prefill     L=512, fp32 throughout, H_I=4, d_I=32, k=64, MLA 4 heads,
                   d_c=64, d_R=16 (key width 80, value width 64); seed 0
  decode_32k       32 single-token decodes, 32768-token contiguous history,
                   FP8 indexer 64x128, k=2048, MLA 128 heads 576/512 bf16,
                   16 planted needle keys per sequence (cosine 0.8); seed 1
  prefill_16k      causal prefill L=16384, same shapes; seed 2
  prefill_64k      causal prefill L=65536, keys = 0.5 * block drift (shared
                   by each 256-token block) + N(0,1) noise; seed 3
  paged_decode     64 decodes, history lengths uniform in [4096, 131072],
                   64-token pages in a randomly permuted pool; seed 4
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK_ROWS = 256
PAGE_SIZE = 64
FP8_MAX = 448.0

T_CTX, T_QI, T_W, T_KI, T_Q, T_KV, T_STRUCT, T_PERM = range(8)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    kind: str                 # "prefill", "decode" or "chunk" (q_per_seq new queries)
    batch: int
    ctx: int                  # prefill length, or fixed decode history
    ctx_range: tuple = None   # (lo, hi) inclusive for ragged decode
    h_i: int = 64
    d_i: int = 128
    fp8: bool = True          # indexer operands in E4M3 (+ fp32 scales)
    top_k: int = 2048
    heads: int = 128
    d_c: int = 512
    d_r: int = 64
    paged: bool = False
    needles: int = 0
    drift_block: int = 0      # >0: keys carry 0.5 * per-block shared drift
    index_scale: float = 1.0  # multiplies every indexer score
    q_per_seq: int = 0        # "chunk": queries per sequence (the last tokens of each history)

    @property
    def d_qk(self) -> int:
        return self.d_c + self.d_r

    @property
    def d_v(self) -> int:
        return self.d_c

    @property
    def sm_scale(self) -> float:
        # 1/sqrt(width of the absorbed per-head q.k product)
        return 1.0 / math.sqrt(self.d_qk)

    @property
    def mla_bf16(self) -> bool:
        return self.fp8


WORKLOADS = {
    "tiny_prefill": Workload("tiny_prefill", 0, "prefill", 1, 512, h_i=4, d_i=32,
                             fp8=False, top_k=64, heads=4, d_c=64, d_r=16),
    "decode_32k": Workload("decode_32k", 1, "decode", 32, 32768, needles=16),
    "prefill_16k": Workload("prefill_16k", 2, "prefill", 1, 16384),
    "prefill_64k": Workload("prefill_64k", 3, "prefill", 1, 65536, drift_block=256),
    "paged_decode": Workload("paged_decode", 4, "decode", 64, 0,
                             ctx_range=(4096, 131072), paged=True),
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(*key) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def _chunked(seed, tid, sub, r0, r1, row_elems, draw):
    """Rows r0..r1-1 of a chunk-seeded tensor, as float32 [r1-r0, row_elems]."""
    out = np.empty((max(r1 - r0, 0), row_elems), dtype=np.float32)
    if r1 <= r0:
        return out
    c0, c1 = r0 // CHUNK_ROWS, (r1 - 1) // CHUNK_ROWS

    def job(c):
        rng = _rng(seed, tid, *sub, c)
        block = draw(rng, CHUNK_ROWS * row_elems).reshape(CHUNK_ROWS, row_elems)
        lo = max(r0, c * CHUNK_ROWS)
        hi = min(r1, (c + 1) * CHUNK_ROWS)
        out[lo - r0:hi - r0] = block[lo - c * CHUNK_ROWS:hi - c * CHUNK_ROWS]

    chunks = range(c0, c1 + 1)
    if len(chunks) == 1:
        job(c0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(job, chunks))
    return out


def _normal(rng, n):
    return rng.standard_normal(n, dtype=np.float32)


def _uniform(rng, n):
    return rng.random(n, dtype=np.float32)


# --------------------------------------------------------------------------
# storage encodings of the inputs (input preparation, not the method)
# --------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def quantize_e4m3_per_token(x: np.ndarray):
    """Per-token FP8 E4M3 storage of float32 rows.

    Token = first axis.  scale = amax / 448 (1 if the token is all zero);
    code = round-to-nearest-even(x / scale) after clamping to +-448 (the cast
    alone would turn out-of-range values into NaN).  Returns (uint8 codes of
    x's shape, float32 scales [tokens]).
    """
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    n = x.shape[0]
    flat = x.reshape(n, -1)
    amax = np.abs(flat).max(axis=1) if flat.shape[1] else np.zeros(n, np.float32)
    scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    y = flat / scale[:, None]
    y = np.clip(y, -FP8_MAX, FP8_MAX).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes.reshape(x.shape), scale


# --------------------------------------------------------------------------
# structure of a workload
# --------------------------------------------------------------------------
@dataclass
class Layout:
    """Batch and cache structure (host arrays, int32)."""
    q_seq_start: np.ndarray          # [B+1]
    k_len: np.ndarray                # [B]
    k_seq_start: np.ndarray          # [B+1] logical rows of each history
    num_queries: int
    max_q_per_seq: int
    max_k_len: int
    page_table: np.ndarray = None    # [B, stride] physical page ids, -1 pad
    num_pages: int = 0
    page_perm: np.ndarray = None     # logical page (in (seq, page) order) -> physical
    needle_pos: list = field(default_factory=list)  # per sequence


def make_layout(wl: Workload) -> Layout:
    if wl.kind == "prefill":
        k_len = np.array([wl.ctx] * wl.batch, dtype=np.int64)
        nq = k_len.copy()
    else:
        if wl.ctx_range is not None:
            lo, hi = wl.ctx_range
            k_len = _rng(wl.seed, T_CTX, 0).integers(lo, hi, size=wl.batch, endpoint=True)
        else:
            k_len = np.array([wl.ctx] * wl.batch, dtype=np.int64)
        nq = np.ones(wl.batch, dtype=np.int64)
        if wl.kind == "chunk":
            nq = np.minimum(k_len, wl.q_per_seq)
    q_seq_start = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    k_seq_start = np.concatenate([[0], np.cumsum(k_len)]).astype(np.int64)
    lay = Layout(q_seq_start=q_seq_start, k_len=k_len.astype(np.int32),
                 k_seq_start=k_seq_start, num_queries=int(nq.sum()),
                 max_q_per_seq=int(nq.max()), max_k_len=int(k_len.max()))
    if wl.paged:
        pages = [(int(n) + PAGE_SIZE - 1) // PAGE_SIZE for n in k_len]
        total = int(sum(pages))
        perm = _rng(wl.seed, T_PERM, 0).permutation(total).astype(np.int32)
        stride = max(pages)
        table = np.full((wl.batch, stride), -1, dtype=np.int32)
        off = 0
        for b, npg in enumerate(pages):
            table[b, :npg] = perm[off:off + npg]
            off += npg
        lay.page_table = table
        lay.num_pages = total
        lay.page_perm = perm
    if wl.needles:
        for b in range(wl.batch):
            pos = _rng(wl.seed, T_STRUCT, 0, b).choice(int(k_len[b]), wl.needles, replace=False)
            lay.needle_pos.append(np.sort(pos))
    return lay


class Synth:
    """Row-regenerable generator of one workload's inputs.

    Query rows are indexed 0..T-1 in batch order; key rows by their logical
    global index k_seq_start[b] + s (the contiguous concatenation of every
    sequence's history, which is also the contiguous cache layout).
    """

    def __init__(self, wl: Workload):
        self.wl = wl
        self.layout = make_layout(wl)

    # ---- float32 draws before any storage encoding ----
    def qi_f32(self, r0, r1):
        wl = self.wl
        return _chunked(wl.seed, T_QI, (), r0, r1, wl.h_i * wl.d_i, _normal).reshape(-1, wl.h_i, wl.d_i)

    def w(self, r0, r1):
        wl = self.wl
        return _chunked(wl.seed, T_W, (), r0, r1, wl.h_i, _uniform)

    def _drift(self, g0, g1, dim, sub):
        """0.5 * D[block] for logical rows g0..g1-1 (one history per batch here)."""
        wl = self.wl
        blk = wl.drift_block
        out = np.empty((g1 - g0, dim), dtype=np.float32)
        for b0 in range(g0 // blk, (g1 - 1) // blk + 1):
            d = _rng(wl.seed, T_STRUCT, sub, b0).standard_normal(dim, dtype=np.float32)
            lo, hi = max(g0, b0 * blk), min(g1, (b0 + 1) * blk)
            out[lo - g0:hi - g0] = np.float32(0.5) * d
        return out

    def ki_f32(self, g0, g1):
        wl = self.wl
        x = _chunked(wl.seed, T_KI, (), g0, g1, wl.d_i, _normal)
        if wl.drift_block:
            x += self._drift(g0, g1, wl.d_i, 1)
        if wl.needles:
            self._plant_needles(x, g0, g1)
        return x

    def _plant_needles(self, x, g0, g1):
        """Replace needle keys by ||k|| (0.8 d + 0.6 e): cosine 0.8 with d.

        d is the unit vector along sum_j w[j] q^I[j] of the sequence's query
        (its head-weighted mean direction); e is a random unit vector
        orthogonal to d; ||k|| is the norm of the replaced draw.
        """
        lay = self.layout
        wl = self.wl
        for b in range(wl.batch):
            base = int(lay.k_seq_start[b])
            if base >= g1 or base + int(lay.k_len[b]) <= g0:
                continue  # no key of this sequence in the range
            qrow = int(lay.q_seq_start[b + 1]) - 1
            qi = self.qi_f32(qrow, qrow + 1)[0].astype(np.float64)
            wv = self.w(qrow, qrow + 1)[0].astype(np.float64)
            d = (wv[:, None] * qi).sum(axis=0)
            d /= np.linalg.norm(d)
            for j, pos in enumerate(lay.needle_pos[b]):
                g = base + int(pos)
                if not (g0 <= g < g1):
                    continue
                e = _rng(wl.seed, T_STRUCT, 2, b, j).standard_normal(wl.d_i)
                e -= np.dot(e, d) * d
                e /= np.linalg.norm(e)
                norm = float(np.linalg.norm(x[g - g0].astype(np.float64)))
                x[g - g0] = (norm * (0.8 * d + 0.6 * e)).astype(np.float32)

    def q_f32(self, r0, r1):
        wl = self.wl
        return _chunked(wl.seed, T_Q, (), r0, r1, wl.heads * wl.d_qk, _normal).reshape(-1, wl.heads, wl.d_qk)

    def kv_f32(self, g0, g1):
        wl = self.wl
        x = _chunked(wl.seed, T_KV, (), g0, g1, wl.d_qk, _normal)
        if wl.drift_block:
            x += self._drift(g0, g1, wl.d_qk, 2)
        return x

    # ---- stored forms ----
    def qi(self, r0, r1):
        """(codes uint8 [n,H_I,d_I], scale f32 [n]) or (f32 [n,H_I,d_I], None)."""
        x = self.qi_f32(r0, r1)
        if self.wl.fp8:
            return quantize_e4m3_per_token(x)
        return x, None

    def ki(self, g0, g1):
        x = self.ki_f32(g0, g1)
        if self.wl.fp8:
            return quantize_e4m3_per_token(x)
        return x, None

    def q(self, r0, r1):
        x = self.q_f32(r0, r1)
        return to_bf16_bits(x) if self.wl.mla_bf16 else x

    def kv(self, g0, g1):
        x = self.kv_f32(g0, g1)
        return to_bf16_bits(x) if self.wl.mla_bf16 else x

    # ---- paged pools ----
    def page_of(self, b, s):
        return int(self.layout.page_table[b, s // PAGE_SIZE])

    def paged_pools(self):
        """Physical pools for the paged layout, with unused slots poisoned.

        Returns (ki_pool [P,64,d_I] uint8, ki_scale_pool [P,64] f32,
        kv_pool [P,64,D_qk] uint16), or for fp32 workloads (ki_pool f32,
        None, kv_pool f32).  Slots past a history's end hold NaN patterns
        (E4M3 0x7F, scale NaN, bfloat16 0x7FC0, fp32 NaN) so that any read of
        them shows up in the results.
        """
        wl, lay = self.wl, self.layout
        assert wl.paged
        P = lay.num_pages
        if wl.fp8:
            ki_pool = np.full((P, PAGE_SIZE, wl.d_i), 0x7F, dtype=np.uint8)
            ks_pool = np.full((P, PAGE_SIZE), np.nan, dtype=np.float32)
            kv_pool = np.full((P, PAGE_SIZE, wl.d_qk), 0x7FC0, dtype=np.uint16)
        else:
            ki_pool = np.full((P, PAGE_SIZE, wl.d_i), np.nan, dtype=np.float32)
            ks_pool = None
            kv_pool = np.full((P, PAGE_SIZE, wl.d_qk), np.nan, dtype=np.float32)
        for b in range(wl.batch):
            n = int(lay.k_len[b])
            base = int(lay.k_seq_start[b])
            step = 16384
            for s0 in range(0, n, step):
                s1 = min(n, s0 + step)
                codes, sc = self.ki(base + s0, base + s1)
                kvb = self.kv(base + s0, base + s1)
                s = np.arange(s0, s1)
                pages = lay.page_table[b, s // PAGE_SIZE]
                slots = s % PAGE_SIZE
                ki_pool[pages, slots] = codes
                if ks_pool is not None:
                    ks_pool[pages, slots] = sc
                kv_pool[pages, slots] = kvb
        return ki_pool, ks_pool, kv_pool
