"""fp32 sparse MLA (dsa_sparse_mla_fwd with DSA_F32) against the float64
oracle, row by row and head by head.

The kernel stages 64 selected rows at a time in LDS, forms logits and P V
with fp32 MFMA tiles of 16 heads, and splits long selections over several
workgroups merged by a combine kernel.  The cases cover every branch of
that design: head counts that are and are not multiples of 16 (1, 5, 16,
33, 64), widths that are and are not multiples of 4 (float4 or scalar
gather), d_v < d_qk, selections of 1, 63, 64, 65 and 2000 slots with -1
padding, a row that selects nothing, one query row (many ranges, the
combine kernel) and 300 rows (one range, no workspace), paged and
contiguous latents, a latent pool that is not 16-byte aligned, and a logit
range wide enough that the running maximum moves across chunks and ranges.

Tolerance: fp32 products and sums of at most 256 terms, softmax in fp32:
max |o - o_ref| <= 1e-4 * max |o_ref| per (row, head), |lse - lse_ref| <=
1e-4 * (1 + |lse_ref|)."""

import zlib

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from sparse_attention_long_fp8_amd import binding as B

pytestmark = pytest.mark.gpu

TOL = 1e-4
PS = 64


def _layout(rng, k_len, paged, gpu):
    """Row of (sequence b, position s) in the pool, and the layout handle."""
    if not paged:
        starts = np.concatenate([[0], np.cumsum(k_len)]).astype(np.int64)
        dev = torch.from_numpy(starts).to(gpu)
        rows = [starts[b] + np.arange(n) for b, n in enumerate(k_len)]
        return B.make_contiguous_layout(dev, int(starts[-1])), dev, rows, int(starts[-1])
    pages = [-(-n // PS) for n in k_len]
    P = sum(pages)
    perm = rng.permutation(P).astype(np.int32)
    stride = max(pages)
    table = -np.ones((len(k_len), stride), np.int32)
    c = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[c:c + n]
        c += n
    dev = torch.from_numpy(table).to(gpu)
    rows = [table[b, np.arange(n) // PS].astype(np.int64) * PS + np.arange(n) % PS for b, n in enumerate(k_len)]
    return B.make_paged_layout(dev, stride, P, PS), dev, rows, P * PS


CASES = {
    # name: (k_len per sequence, queries per sequence, heads, d_qk, d_v, k, paged, misalign, sm_scale or None)
    "one_row_many_ranges": ([3000], [1], 16, 256, 256, 512, False, False, None),
    "ragged_small_heads": ([40, 700, 130], [1, 2, 1], 5, 7, 3, 65, False, False, None),
    "paged_h64": ([900, 2500], [20, 20], 64, 256, 200, 300, True, False, None),
    "many_rows_one_range": ([600] * 3, [100] * 3, 33, 80, 64, 64, False, False, None),
    "unaligned_pool": ([800], [3], 16, 128, 128, 63, False, True, None),
    "k1": ([50, 60], [2, 2], 1, 12, 12, 1, True, False, None),
    "wide_logits_k2000": ([5000], [2], 16, 64, 64, 2000, False, False, 1.0),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_f32_mla_matches_oracle(gpu, name):
    k_len, q_per, H, d_qk, d_v, k, paged, misalign, scale = CASES[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    sm_scale = scale if scale is not None else 1.0 / np.sqrt(d_qk)
    ly, ly_keep, rows, n_rows = _layout(rng, k_len, paged, gpu)
    pool = rng.standard_normal((n_rows, d_qk)).astype(np.float32)
    seq_of = np.repeat(np.arange(len(k_len)), q_per)
    T = len(seq_of)
    q = rng.standard_normal((T, H, d_qk)).astype(np.float32)
    idx = -np.ones((T, k), np.int32)
    for t, b in enumerate(seq_of):
        n = k_len[b]
        m = min(k, n) if t % 3 else max(min(k, n) - 7, 1)   # some rows leave -1 padding
        idx[t, :m] = np.sort(rng.choice(n, m, replace=False))
    if T >= 3:
        idx[T // 2] = -1                                     # a row that selects nothing
    q_seq_start = np.concatenate([[0], np.cumsum(q_per)]).astype(np.int32)
    t_ = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
    qs_d, kl_d = t_(q_seq_start), t_(np.asarray(k_len, np.int32))
    bt = B.make_batch(qs_d, kl_d, len(k_len), T, max(q_per), max(k_len))
    if misalign:   # pool starts 4 bytes past a 16-byte boundary
        buf = torch.zeros(pool.size + 4, dtype=torch.float32, device=gpu)
        kv = buf[1:1 + pool.size].view(n_rows, d_qk)
        kv.copy_(t_(pool))
        assert kv.data_ptr() % 16 == 4
    else:
        kv = t_(pool)
    out = torch.full((T, H, d_v), float("nan"), device=gpu)
    lse = torch.full((T, H), float("nan"), device=gpu)
    nb = B.dsa_sparse_mla_workspace_size(bt, B.DSA_F32, H, d_qk, d_v, k)
    ws = torch.empty(max(nb, 1) + 256, dtype=torch.uint8, device=gpu)
    base = ws.data_ptr() + (-ws.data_ptr()) % 256
    B.dsa_sparse_mla_fwd(bt, ly, B.DSA_F32, H, d_qk, d_v, t_(q), kv, t_(idx), k, sm_scale, out, lse, base, nb)
    torch.cuda.synchronize()
    got_o, got_l = out.cpu().numpy(), lse.cpu().numpy()
    assert not np.isnan(got_o).any() and not np.isnan(got_l).any()
    for t, b in enumerate(seq_of):
        o_ref, l_ref = O.sparse_mla(q[t], pool[rows[b]], idx[t], d_v, sm_scale)
        if (idx[t] < 0).all():
            assert (got_o[t] == 0).all() and np.isneginf(got_l[t]).all(), "row %d: empty selection" % t
            continue
        err = np.abs(got_o[t] - o_ref).max(axis=1) / np.abs(o_ref).max(axis=1)
        assert err.max() <= TOL, "row %d head %d: %.3g" % (t, int(err.argmax()), err.max())
        assert (np.abs(got_l[t] - l_ref) <= TOL * (1 + np.abs(l_ref))).all(), "row %d: lse" % t
