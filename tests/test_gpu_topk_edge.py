"""Top-k on crafted score rows, bit-exact against the oracle's selection:
heavy ties (small bins resolved by ranking, large ones by radix digits), a
constant row (the whole row is one bin, past the candidate list), signed
zeros, all-negative rows, rows longer than the LDS row cache, rows
shorter than k, ReLU rows that are half exact zeros, k above 2048, ties
spread over the parts of rows longer than 32768 (selected in two passes when
the batch has few rows), decode-like rows of few-row batches at lengths
around 8192, 12288 and 32768, rows where only every 32nd score is large, rows
with -inf scores, heavy ties at the k-th score, and crafted rows of 16385 to 32768 scores in a
small batch with k = 4096 and 4097 (ties across position 16384, ragged
lengths).  Each row is its own sequence, so n_t = k_len[t]; entries
past n_t are NaN and must never be read."""

import zlib

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from sparse_attention_long_fp8_amd import binding as B

pytestmark = pytest.mark.gpu


def _rows(kind, rng):
    if kind == "ties_small_bins":
        return [rng.integers(0, 4000, 5000).astype(np.float32) for _ in range(6)], 300
    if kind == "ties_few_values":
        return [rng.integers(0, 3, 20000).astype(np.float32) for _ in range(3)], 2048
    if kind == "constant":
        return [np.full(4000, 1.5, np.float32), np.full(3000, -2.0, np.float32)], 100
    if kind == "signed_zero":
        r = rng.choice(np.array([0.0, -0.0, 1.0, -1.0], np.float32), 3000)
        return [r, np.where(rng.random(3000) < 0.5, np.float32(-0.0), np.float32(0.0))], 64
    if kind == "all_negative":
        return [-rng.random(9000).astype(np.float32) - 1.0 for _ in range(2)], 512
    if kind == "long_rows":
        return [rng.integers(0, 1000, 70000).astype(np.float32), rng.standard_normal(100000).astype(np.float32)], 2048
    if kind == "relu_zeros":   # about half the row is exactly 0 (one histogram bin)
        return [np.maximum(rng.standard_normal(16384), 0).astype(np.float32) for _ in range(2)], 512
    if kind == "k_above_staging":   # more outputs than the LDS staging holds: direct stores
        return [rng.standard_normal(20000).astype(np.float32), rng.integers(0, 50, 40000).astype(np.float32)], 3000
    if kind == "long_ties":   # ties across the 32768-long parts of a two-pass selection
        return [np.full(70000, 2.5, np.float32), rng.integers(0, 4, 90000).astype(np.float32)], 5000
    if kind == "mid_ties":     # ties across position 16384, ragged rows
        return [np.full(30000, 0.5, np.float32), rng.integers(0, 4, 25000).astype(np.float32),
                rng.standard_normal(1000).astype(np.float32), rng.integers(0, 2, 16385).astype(np.float32),
                np.concatenate([np.zeros(16384, np.float32), np.ones(8000, np.float32)])], 4096
    if kind == "mid_k_limit":
        return [np.full(30000, 0.5, np.float32), rng.integers(0, 4, 25000).astype(np.float32)], 4097
    if kind == "decode_lengths":   # decode rows of few-row batches, around 4k-multiples
        return [rng.standard_normal(n).astype(np.float32) for n in (8191, 8192, 8193, 12288, 12289, 32768,
                                                                     32769, 131072)], 2048
    if kind == "strided_high":   # every 32nd score is large, the rest small
        n = 65536
        r = rng.random(n).astype(np.float32)
        r[(np.arange(2048, dtype=np.int64) * n) // 2048] += 10.0
        return [r, rng.standard_normal(n).astype(np.float32)], 4000
    if kind == "infinities":   # -inf scores, often and rarely
        a = rng.standard_normal(40000).astype(np.float32)
        a[::7] = -np.inf
        b = rng.standard_normal(40000).astype(np.float32)
        b[(np.arange(2048, dtype=np.int64) * 40000) // 2048 + 1] = -np.inf
        return [a, b], 2048
    if kind == "threshold_ties":   # the k-th score has hundreds of equal copies
        return [rng.integers(0, 40, 32768).astype(np.float32), rng.integers(0, 200, 50000).astype(np.float32)], 2048
    if kind == "short_rows":
        return [rng.standard_normal(n).astype(np.float32) for n in (1, 10, 63, 64, 65)], 64
    raise KeyError(kind)


@pytest.mark.parametrize("kind", ["ties_small_bins", "ties_few_values", "constant", "signed_zero",
                                  "all_negative", "long_rows", "short_rows", "relu_zeros", "k_above_staging",
                                  "long_ties", "mid_ties", "mid_k_limit", "decode_lengths",
                                  "strided_high", "infinities", "threshold_ties"])
def test_topk_crafted_rows(kind, gpu):
    print("\n[topk-edge] %s" % kind, flush=True)
    rng = np.random.default_rng(zlib.crc32(kind.encode()))
    rows, k = _rows(kind, rng)
    T = len(rows)
    ns = [len(r) for r in rows]
    ld = (max(ns) + 3) // 4 * 4
    scores = np.full((T, ld), np.nan, np.float32)
    for t, r in enumerate(rows):
        scores[t, :len(r)] = r
    q_seq_start = torch.arange(T + 1, dtype=torch.int32, device=gpu)
    k_len = torch.tensor(ns, dtype=torch.int32, device=gpu)
    batch = B.make_batch(q_seq_start, k_len, T, T, 1, max(ns))
    d_scores = torch.from_numpy(scores).to(gpu)
    idx = torch.full((T, k), -7, dtype=torch.int32, device=gpu)
    nb = B.dsa_topk_workspace_size(batch, k)   # rows past 32768 in a small batch: two passes
    ws = torch.empty(nb + 256, dtype=torch.uint8, device=gpu) if nb else None
    base = ws.data_ptr() + (-ws.data_ptr()) % 256 if nb else None
    B.dsa_topk(batch, d_scores, ld, k, idx, base, nb)
    torch.cuda.synchronize()
    got = idx.cpu().numpy().astype(np.int64)
    for t, r in enumerate(rows):
        want = O.topk_indices(r.astype(np.float64), k)
        assert np.array_equal(got[t], want), "%s row %d (n=%d): top-k differs" % (kind, t, len(r))
