"""bf16 sparse MLA over batches of many sequences, against the float64
oracle row by row.

The attention kernel finds each query row's sequence from q_seq_start with a
wave-wide search that reads 64 entries a round.  These batches need one
round with entries past the end of the array (65 sequences), two rounds (300)
and three (5000).  Many sequences have no query, so q_seq_start holds long
runs of equal entries, and the row must land in the sequence that owns it.
A wrong sequence reads another sequence's key rows and shows up as an
attention error.  The batches also cover 32, 64 and 128 heads, contiguous
and paged latents, selections split over several ranges (with the merge),
-1 padding, and a row that selects nothing.

Tolerance: the bf16 attention bars of the parity tests (max |o - o_ref| /
max |o_ref| <= 2e-2 per row; |lse - lse_ref| <= 1e-2)."""

import zlib

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from sparse_attention_long_fp8_amd import binding as B

pytestmark = pytest.mark.gpu

ATTN_TOL, LSE_TOL = 2e-2, 1e-2
D_QK, D_V, PS = 576, 512, 64

CASES = {
    # name: (sequences, queries of sequence b, history range, k, heads, paged)
    "s65_h64_split": (65, lambda b: 0 if b % 13 == 5 else 1, (300, 900), 512, 64, False),
    "s300_h128_paged": (300, lambda b: 0 if b % 3 == 0 else 1, (60, 400), 256, 128, True),
    "s5000_h32": (5000, lambda b: 3 if b == 4321 else (1 if b % 25 == 7 else 0), (4, 24), 16, 32, False),
}


def _bf16_bits(rng, shape):
    return (rng.standard_normal(shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("name", sorted(CASES))
def test_many_sequences_match_oracle(gpu, name):
    S, q_of, (lo, hi), k, H, paged = CASES[name]
    print("\n[many-seqs] %s" % name, flush=True)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    q_per = np.array([q_of(b) for b in range(S)], np.int32)
    k_len = rng.integers(lo, hi, S).astype(np.int32)
    k_len = np.maximum(k_len, q_per)
    T = int(q_per.sum())
    seq_of = np.repeat(np.arange(S), q_per)
    q_seq_start = np.concatenate([[0], np.cumsum(q_per)]).astype(np.int32)
    t_ = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
    if paged:
        pages = -(-k_len // PS)
        P = int(pages.sum())
        perm = rng.permutation(P).astype(np.int32)
        stride = int(pages.max())
        table = -np.ones((S, stride), np.int32)
        starts = np.concatenate([[0], np.cumsum(pages)])
        for b in range(S):
            table[b, :pages[b]] = perm[starts[b]:starts[b + 1]]
        keep = t_(table)
        layout = B.make_paged_layout(keep, stride, P, PS)
        n_rows = P * PS
        rows_of = lambda b: table[b, np.arange(k_len[b]) // PS].astype(np.int64) * PS + np.arange(k_len[b]) % PS
    else:
        kss = np.concatenate([[0], np.cumsum(k_len)[:-1]]).astype(np.int64)
        keep = t_(kss)
        n_rows = int(k_len.sum())
        layout = B.make_contiguous_layout(keep, n_rows)
        rows_of = lambda b: kss[b] + np.arange(k_len[b])
    kv_bits = _bf16_bits(rng, (n_rows, D_QK))
    q_bits = _bf16_bits(rng, (T, H, D_QK))
    idx = -np.ones((T, k), np.int32)
    for t, b in enumerate(seq_of):
        n = int(k_len[b] - q_per[b] + (t - q_seq_start[b]) + 1)   # causal candidates of row t
        m = min(k, n) if t % 4 else max(min(k, n) - 5, 1)        # some rows leave -1 padding
        idx[t, :m] = np.sort(rng.choice(n, m, replace=False))
    idx[T // 2] = -1                                              # a row that selects nothing
    qs_d, kl_d = t_(q_seq_start), t_(k_len)   # held until the kernels have run
    bt = B.make_batch(qs_d, kl_d, S, T, int(q_per.max()), int(k_len.max()))
    as_bf16 = lambda bits: t_(bits.view(np.int16)).view(torch.bfloat16)
    q, kv = as_bf16(q_bits), as_bf16(kv_bits)
    out = torch.full((T, H, D_V), float("nan"), dtype=torch.bfloat16, device=gpu)
    lse = torch.full((T, H), float("nan"), device=gpu)
    nb = B.dsa_sparse_mla_workspace_size(bt, B.DSA_BF16, H, D_QK, D_V, k)
    ws = torch.empty(max(nb, 1) + 256, dtype=torch.uint8, device=gpu)
    base = ws.data_ptr() + (-ws.data_ptr()) % 256
    B.dsa_sparse_mla_fwd(bt, layout, B.DSA_BF16, H, D_QK, D_V, q, kv, t_(idx), k, D_QK ** -0.5, out, lse,
                         base, nb)
    torch.cuda.synchronize()
    got_o = out.float().cpu().numpy().astype(np.float64)
    got_l = lse.cpu().numpy()
    for t, b in enumerate(seq_of):
        o_ref, l_ref = O.sparse_mla(O.decode_bf16(q_bits[t]), O.decode_bf16(kv_bits[rows_of(b)]), idx[t], D_V,
                                    D_QK ** -0.5)
        if (idx[t] < 0).all():
            assert (got_o[t] == 0).all() and np.isneginf(got_l[t]).all(), "row %d: empty selection" % t
            continue
        assert not np.isnan(got_o[t]).any(), "row %d (sequence %d): NaN" % (t, b)
        err = np.abs(got_o[t] - o_ref).max() / np.abs(o_ref).max()
        assert err <= ATTN_TOL, "row %d (sequence %d): attention error %.3g" % (t, b, err)
        assert np.abs(got_l[t] - l_ref).max() <= LSE_TOL, "row %d (sequence %d): lse" % (t, b)
