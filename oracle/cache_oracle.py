"""Plain CPU oracle for the decode-step cache append.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test-suite and the benchmark's CPU leg use it.
It shares no code with the HIP library.

What it computes.  Before a decoding step scores its history, the new token's
entries must be in the caches the step reads: its indexer key, stored in FP8
with one fp32 scale per token ("DeepSeek Sparse Attention DSA Architecture
Guide", "Stage 1: The Lightning Indexer", item 1: the indexer's intermediate
states are FP8), and its compressed latent row ("Stage 2: Fine-Grained Token
Selection", the cached c^KV the gather reads).  "Sparse Attention
Architectures for Long-Context Inference: Evolution and Engineering
Practices", section 6 ("incremental inference adaptation"), names this
per-step cache update; "Sparse Attention in Large Language Models:
Architecture Evolution and Engineering Practice", section 4.1, recommends
paged KV storage, so both pools may be paged (64-token pages).

Readings (the pages fix none of these):
  * one scale per token: scale = amax / 448 in fp32, or 1 for an all-zero
    row; code = round-to-nearest-even of (x / scale) in fp32 after clamping
    to +-448, in OCP E4M3 (448 is its largest finite value);
  * a quantised code is an integer decided by floating point, so this oracle
    takes the decision in the kernel's precision (fp32 division and clamp),
    and rounds by an exact nearest search over the format's values;
  * the latent row is stored unchanged (bf16 in, bf16 out).
"""

from __future__ import annotations

import numpy as np

from .dsa_oracle import E4M3_TABLE

__all__ = ["FP8_MAX", "encode_e4m3_rne", "quantize_token", "cache_row", "cache_append"]

FP8_MAX = 448.0

# finite non-negative E4M3 values, codes 0x00 .. 0x7E, strictly increasing
_POS_VALUES = E4M3_TABLE[:0x7F]


def encode_e4m3_rne(y: np.ndarray) -> np.ndarray:
    """float32 values already within [-448, 448] -> E4M3 codes (uint8).

    The magnitude goes to the nearest finite E4M3 value; when it lies exactly
    halfway between two, the one with the even code (mantissa LSB 0) wins.
    The sign bit is copied, so -0.0 and negative values that round to zero
    give 0x80.
    """
    y = np.asarray(y, dtype=np.float32)
    if np.isnan(y).any() or (np.abs(y) > FP8_MAX).any():
        raise ValueError("encode_e4m3_rne: values must be finite and within +-448")
    a = np.abs(y).astype(np.float64).ravel()
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a (a <= 448 = last)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    nearest = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    code = np.where(tie, np.where(lo % 2 == 0, lo, hi), nearest)
    code = np.where(hi == 0, 0, code)  # a == 0
    out = code.astype(np.uint8)
    out |= (np.signbit(y).ravel().astype(np.uint8) << 7)
    return out.reshape(y.shape)


def quantize_token(x: np.ndarray):
    """One token's fp32 key -> (E4M3 codes, fp32 scale), per the readings above."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    scale = np.float32(amax / np.float32(FP8_MAX)) if amax > 0 else np.float32(1.0)
    y = (x / scale).astype(np.float32)
    y = np.minimum(np.maximum(y, np.float32(-FP8_MAX)), np.float32(FP8_MAX))
    return encode_e4m3_rne(y), scale


def cache_row(layout: dict, b: int, p: int):
    """Pool index of logical position p of sequence b.

    Paged layout (``page_table`` [B, stride], ``page_size``): page
    page_table[b, p // page_size], slot p % page_size, returned as a
    (page, slot) pair.  Contiguous layout (``k_seq_start`` [B+1]): flat row
    k_seq_start[b] + p, returned as a 1-tuple.
    """
    if layout.get("paged"):
        ps = int(layout["page_size"])
        page = int(layout["page_table"][b][p // ps])
        if page < 0:
            raise ValueError("position %d of sequence %d has no page" % (p, b))
        return (page, p % ps)
    return (int(layout["k_seq_start"][b]) + p,)


def cache_append(layout: dict, seq, pos, k_new, latent_new, k_pool, ksc_pool, latent_pool):
    """Return copies of the three pools with every new token written.

    Token i of the call belongs to sequence seq[i] at logical position
    pos[i]; its key k_new[i] (fp32) is quantised per token into k_pool /
    ksc_pool, and its latent row latent_new[i] (bf16 bit patterns) is copied
    into latent_pool.  ``latent_new`` / ``latent_pool`` may be None (keys
    only).  Positions are distinct, so the order of tokens does not matter.
    """
    k_pool = np.array(k_pool, copy=True)
    ksc_pool = np.array(ksc_pool, copy=True)
    latent_pool = None if latent_pool is None else np.array(latent_pool, copy=True)
    for i in range(len(seq)):
        where = cache_row(layout, int(seq[i]), int(pos[i]))
        codes, scale = quantize_token(k_new[i])
        k_pool[where] = codes
        ksc_pool[where] = scale
        if latent_pool is not None:
            latent_pool[where] = latent_new[i]
    return k_pool, ksc_pool, latent_pool
