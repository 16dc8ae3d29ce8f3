"""Pins for the CPU oracle: each check compares it with something other than
itself -- a library routine, brute force, a closed form or a hand-derived
fixture -- so that a dropped term, a wrong sign, index or operand order in
the oracle fails at least one of them."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- formats
def test_e4m3_table_matches_torch_for_all_256_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = O.decode_e4m3(np.arange(256, dtype=np.uint8))
    nan_ref, nan_mine = np.isnan(ref), np.isnan(mine)
    assert (nan_ref == nan_mine).all()
    assert set(np.nonzero(nan_mine)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan_ref], mine[~nan_mine])


def test_e4m3_spot_values():
    t = O.E4M3_TABLE
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x38] == 1.0
    assert t[0x00] == 0.0 and math.copysign(1, t[0x80]) == -1


# every 16-bit pattern is decoded, the signalling NaNs too, whose widening
# numpy reports as an invalid operation
@pytest.mark.filterwarnings("ignore:invalid value encountered in cast:RuntimeWarning")
def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = O.decode_bf16(bits)
    ok = ~np.isnan(ref)
    assert (np.isnan(mine) == ~ok).all()
    assert np.array_equal(ref[ok], mine[ok])


def test_dequant_is_exact_product():
    codes = np.array([[0x38, 0x7E], [0x01, 0xB8]], dtype=np.uint8)
    scale = np.array([0.5, 3.0], dtype=np.float32)
    got = O.dequant_e4m3(codes, scale)
    assert np.array_equal(got, np.array([[0.5, 224.0], [3.0 * 2 ** -9, -3.0]]))


# ---------------------------------------------------------------- bookkeeping
def test_query_rows_prefill_and_decode():
    # prefill: 3 queries over 3 keys -> positions 0,1,2
    assert O.query_rows([0, 3], [3]) == [(0, 0, 1), (0, 1, 2), (0, 2, 3)]
    # decode: one query per sequence at the last position
    assert O.query_rows([0, 1, 2], [5, 9]) == [(0, 4, 5), (1, 8, 9)]
    # chunked prefill: 2 new queries after 4 cached keys
    assert O.query_rows([0, 2], [6]) == [(0, 4, 5), (0, 5, 6)]
    with pytest.raises(ValueError):
        O.query_rows([0, 4], [3])


def test_unpage_matches_contiguous():
    rng = np.random.default_rng(3)
    n, page = 300, 64
    logical = rng.standard_normal((n, 5))
    npages = (n + page - 1) // page
    perm = rng.permutation(npages + 3)[:npages]          # spare pages unused
    pool = np.full((npages + 3, page, 5), np.nan)
    for s in range(n):
        pool[perm[s // page], s % page] = logical[s]
    table = np.concatenate([perm, [-1, -1]])
    assert np.array_equal(O.unpage(pool, table, n, page), logical)


# ---------------------------------------------------------------- indexer
def test_indexer_hand_fixture():
    g = _load("indexer_hand.json")
    got = O.indexer_scores(np.array(g["q"], float), np.array(g["w"]), np.array(g["keys"], float), g["scale"])
    assert np.array_equal(got, np.array(g["expected"]))


def test_indexer_single_head_equals_page_module():
    """H_I = 1, w = 1, scale = 1/sqrt(d_I) is the page's LightningIndexer:
    relu(bmm(q, k^T) * scale), evaluated here with torch in float64."""
    rng = np.random.default_rng(11)
    d_i, n = 32, 77
    q = rng.standard_normal((1, d_i))
    k = rng.standard_normal((n, d_i))
    qt = torch.from_numpy(q).view(1, 1, d_i)
    kt = torch.from_numpy(k).view(1, n, d_i)
    ref = torch.relu(torch.bmm(qt, kt.transpose(1, 2).contiguous()) * (1.0 / d_i ** 0.5)).view(n).numpy()
    got = O.indexer_scores(q, np.ones(1), k, 1.0 / math.sqrt(d_i))
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_indexer_brute_force_loops():
    rng = np.random.default_rng(5)
    h, d, n = 3, 4, 9
    q = rng.standard_normal((h, d))
    w = rng.uniform(-1, 1, h)
    k = rng.standard_normal((n, d))
    want = []
    for s in range(n):
        total = 0.0
        for j in range(h):
            dot = 0.0
            for x in range(d):
                dot += q[j, x] * k[s, x]
            total += w[j] * (dot if dot > 0 else 0.0)
        want.append(0.25 * total)
    np.testing.assert_allclose(O.indexer_scores(q, w, k, 0.25), want, rtol=1e-13, atol=1e-14)


def test_indexer_closed_forms():
    rng = np.random.default_rng(9)
    h, d, n = 4, 8, 50
    q = rng.standard_normal((h, d))
    k = rng.standard_normal((n, d))
    w1, w2 = rng.uniform(0, 1, h), rng.uniform(0, 1, h)
    # zero query -> all scores zero
    assert np.array_equal(O.indexer_scores(np.zeros((h, d)), w1, k), np.zeros(n))
    # linear in w
    np.testing.assert_allclose(O.indexer_scores(q, w1 + w2, k),
                               O.indexer_scores(q, w1, k) + O.indexer_scores(q, w2, k), rtol=1e-12)
    # non-negative for non-negative weights
    assert (O.indexer_scores(q, w1, k) >= 0).all()
    # doubling one key's FP8 scale doubles exactly that key's score
    codes = np.random.default_rng(2).integers(0, 0x7E, size=(n, d)).astype(np.uint8)
    sc = np.ones(n, np.float32)
    base = O.indexer_scores(q, w1, O.dequant_e4m3(codes, sc))
    sc2 = sc.copy()
    sc2[17] = 2.0
    doubled = O.indexer_scores(q, w1, O.dequant_e4m3(codes, sc2))
    assert doubled[17] == 2 * base[17]
    assert np.array_equal(np.delete(doubled, 17), np.delete(base, 17))


# ---------------------------------------------------------------- top-k
def _scores_from_json(vals):
    return np.array([-0.0 if v == "-0" else float(v) for v in vals])


def test_topk_hand_fixture():
    g = _load("topk_hand.json")
    s = _scores_from_json(g["scores"])
    for case in g["cases"]:
        assert O.topk_indices(s, case["k"]).tolist() == case["expected"], case["why"]


def _check_topk_brute(s, k, idx):
    n = len(s)
    m = min(k, n)
    chosen = idx[:m]
    assert (idx[m:] == -1).all()
    assert (np.diff(chosen) > 0).all() and chosen.min() >= 0 and chosen.max() < n
    rest = np.setdiff1d(np.arange(n), chosen)
    if m and rest.size:
        tau = s[chosen].min()
        assert s[rest].max() <= tau
        # at the threshold value, the chosen equal positions are the lowest ones
        eq = np.nonzero(s == tau)[0]
        eq_chosen = np.intersect1d(eq, chosen)
        assert np.array_equal(eq_chosen, eq[:eq_chosen.size])


def test_topk_brute_force_properties_with_many_ties():
    rng = np.random.default_rng(1)
    for trial in range(300):
        n = int(rng.integers(1, 60))
        k = int(rng.integers(1, 70))
        s = rng.integers(0, 5, size=n).astype(float)
        _check_topk_brute(s, k, O.topk_indices(s, k))


def test_topk_special_cases():
    s = np.random.default_rng(0).standard_normal(10)
    assert O.topk_indices(s, 10).tolist() == list(range(10))
    assert O.topk_indices(s, 12).tolist() == list(range(10)) + [-1, -1]
    assert O.topk_indices(np.full(20, 1.5), 6).tolist() == list(range(6))
    with pytest.raises(ValueError):
        O.topk_indices(np.array([1.0, np.nan]), 1)


def test_topk_commutes_across_tiles():
    """Per-key separable scores: top-k of a row equals top-k over the union
    of each tile's own top-k (Stage 1, item 3 of the DSA guide)."""
    rng = np.random.default_rng(4)
    for trial in range(50):
        n = int(rng.integers(50, 400))
        k = int(rng.integers(1, 40))
        s = rng.integers(0, 30, size=n).astype(float)
        cut = int(rng.integers(1, n))
        a = O.topk_indices(s[:cut], k)
        b = O.topk_indices(s[cut:], k)
        cand = np.concatenate([a[a >= 0], b[b >= 0] + cut])
        merged = O.topk_indices(s[cand], k)
        merged = np.sort(cand[merged[merged >= 0]])
        full = O.topk_indices(s, k)
        assert np.array_equal(full[full >= 0], merged)


# ---------------------------------------------------------------- sparse MLA
def test_mla_hand_fixture():
    g = _load("mla_hand.json")
    kv = np.array(g["kv"], float)
    q = np.array([[0.0, math.log(3.0)], [1.0, 0.0]])
    o, lse = O.sparse_mla(q, kv, np.array([0, 1]), g["d_v"], g["sm_scale"])
    assert abs(o[0, 0] - 17.5) < 1e-12 and abs(lse[0] - math.log(4.0)) < 1e-12
    assert abs(o[1, 0] - (10 + 10 / (1 + math.exp(-10)))) < 1e-12
    assert abs(lse[1] - (20 + math.log1p(math.exp(-10)))) < 1e-12
    # order of the selected positions and -1 padding do not matter
    o2, lse2 = O.sparse_mla(q, kv, np.array([1, -1, 0, -1]), 1, 1.0)
    np.testing.assert_allclose(o2, o, rtol=1e-15)
    np.testing.assert_allclose(lse2, lse, rtol=1e-15)


def test_dense_causal_mla_matches_torch_sdpa():
    """The independent dense routine against torch's causal attention (float64)."""
    rng = np.random.default_rng(8)
    T, H, D, Dv = 12, 3, 6, 4
    q = rng.standard_normal((T, H, D))
    kv = rng.standard_normal((T, D))
    sc = 1 / math.sqrt(D)
    o, lse = O.dense_causal_mla(q, kv, Dv, sc)
    qt = torch.from_numpy(q).permute(1, 0, 2).contiguous()            # [H, T, D]
    kt = torch.from_numpy(kv).expand(H, T, D).contiguous()
    vt = torch.from_numpy(kv[:, :Dv]).expand(H, T, Dv).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=sc)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    logits = torch.bmm(qt, kt.transpose(1, 2).contiguous()) * sc
    mask = torch.triu(torch.ones(T, T, dtype=torch.bool), 1)
    ref_lse = torch.logsumexp(logits.masked_fill(mask, float("-inf")), dim=-1).T.numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_sparse_with_k_at_least_context_is_dense():
    rng = np.random.default_rng(12)
    T, H, D, Dv, Hi, Di = 20, 2, 10, 8, 3, 4
    q = rng.standard_normal((T, H, D))
    kv = rng.standard_normal((T, D))
    qi = rng.standard_normal((T, Hi, Di))
    ki = rng.standard_normal((T, Di))
    w = rng.uniform(0, 1, (T, Hi))
    o_d, lse_d = O.dense_causal_mla(q, kv, Dv, 0.3)
    for t in range(T):
        s, idx, o, lse = O.forward_row(qi[t], w[t], ki, q[t], kv, t + 1, T + 5, 1.0, Dv, 0.3)
        assert idx[:t + 1].tolist() == list(range(t + 1))
        np.testing.assert_allclose(o, o_d[t], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, lse_d[t], rtol=1e-12, atol=1e-12)


def test_mla_closed_forms():
    rng = np.random.default_rng(13)
    H, D, Dv, n = 3, 7, 5, 30
    kv = rng.standard_normal((n, D))
    q = rng.standard_normal((H, D))
    # a single selected row: output is that row's value part, lse is its logit
    o, lse = O.sparse_mla(q, kv, np.array([4, -1, -1]), Dv, 0.7)
    assert np.array_equal(o, np.tile(kv[4, :Dv], (H, 1)))
    np.testing.assert_allclose(lse, 0.7 * (q @ kv[4]), rtol=1e-14)
    # zero query: uniform weights -> mean of the selected value rows, lse = log m
    sel = np.array([1, 5, 9, 22])
    o, lse = O.sparse_mla(np.zeros((H, D)), kv, sel, Dv, 0.7)
    np.testing.assert_allclose(o, np.tile(kv[sel, :Dv].mean(0), (H, 1)), rtol=1e-13)
    np.testing.assert_allclose(lse, np.log(4.0), rtol=1e-14)
    # permuting the selected positions changes nothing beyond rounding
    o1, l1 = O.sparse_mla(q, kv, sel, Dv, 0.7)
    o2, l2 = O.sparse_mla(q, kv, sel[::-1], Dv, 0.7)
    np.testing.assert_allclose(o1, o2, rtol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)
    # nothing selected
    o, lse = O.sparse_mla(q, kv, np.array([-1, -1]), Dv, 0.7)
    assert (o == 0).all() and np.isneginf(lse).all()
