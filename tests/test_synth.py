"""Checks of the seeded input generator: determinism, row regeneration,
storage encodings, workload structure (needles, drift, pages)."""

import numpy as np

from oracle import dsa_oracle as O
from sparse_attention_long_fp8_amd import synth


def test_rows_regenerate_independently():
    s = synth.Synth(synth.WORKLOADS["prefill_16k"])
    whole = s.q_f32(200, 800)
    part = s.q_f32(517, 530)
    assert np.array_equal(whole[317:330], part)
    assert np.array_equal(s.ki_f32(0, 300)[255:260], s.ki_f32(255, 260))


def test_e4m3_quantiser_round_trip():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((64, 3, 16)).astype(np.float32) * rng.uniform(0.01, 100, (64, 1, 1)).astype(np.float32)
    x[5] = 0.0
    codes, scale = synth.quantize_e4m3_per_token(x)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    assert scale[5] == 1.0 and (codes[5] == 0).all()
    back = O.dequant_e4m3(codes, scale)
    for t in range(64):
        if t == 5:
            continue
        amax = np.abs(x[t]).max()
        # the largest magnitude maps to +-448 exactly
        assert np.abs(O.decode_e4m3(codes[t])).max() == 448.0
        y = x[t].astype(np.float64)
        big = np.abs(y) >= 2.0 ** -6 * amax / 448 * 8   # normal range of the code
        err = np.abs(back[t] - y)
        # round to nearest with a 3-bit mantissa: relative error <= 2^-4
        assert (err[big] <= np.abs(y[big]) * 2.0 ** -4 * 1.0001).all()
        assert (err <= amax / 448 * 2.0 ** -9 * 1.0001 + np.abs(y) * 2.0 ** -4).all()


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], dtype=np.float32)
    bits = synth.to_bf16_bits(x)
    assert O.decode_bf16(bits).tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5]


def test_layouts():
    lay = synth.make_layout(synth.WORKLOADS["decode_32k"])
    assert lay.num_queries == 32 and (lay.k_len == 32768).all()
    assert lay.q_seq_start.tolist() == list(range(33))
    lay = synth.make_layout(synth.WORKLOADS["prefill_64k"])
    assert lay.num_queries == 65536 and lay.max_q_per_seq == 65536
    pw = synth.WORKLOADS["paged_decode"]
    lay = synth.make_layout(pw)
    assert lay.k_len.min() >= 4096 and lay.k_len.max() <= 131072
    pages = (lay.k_len.astype(int) + 63) // 64
    assert lay.num_pages == pages.sum()
    used = lay.page_table[lay.page_table >= 0]
    assert np.array_equal(np.sort(used), np.arange(lay.num_pages))   # a permutation
    for b in range(pw.batch):
        assert (lay.page_table[b, :pages[b]] >= 0).all() and (lay.page_table[b, pages[b]:] == -1).all()


def test_needles_have_cosine_point_eight():
    s = synth.Synth(synth.WORKLOADS["decode_32k"])
    lay = s.layout
    for b in (0, 7):
        qi = s.qi_f32(b, b + 1)[0].astype(np.float64)
        w = s.w(b, b + 1)[0].astype(np.float64)
        d = (w[:, None] * qi).sum(0)
        d /= np.linalg.norm(d)
        base = int(lay.k_seq_start[b])
        for pos in lay.needle_pos[b][:4]:
            k = s.ki_f32(base + int(pos), base + int(pos) + 1)[0].astype(np.float64)
            assert abs(np.dot(k, d) / np.linalg.norm(k) - 0.8) < 1e-5


def test_needles_recalled_by_oracle():
    """Every planted needle is among the oracle's top-2048 positions."""
    wl = synth.WORKLOADS["decode_32k"]
    s = synth.Synth(wl)
    lay = s.layout
    for b in (0, 13, 31):
        codes, sc = s.qi(b, b + 1)
        qi = O.dequant_e4m3(codes, sc)[0]
        w = s.w(b, b + 1)[0]
        base = int(lay.k_seq_start[b])
        kc, ks = s.ki(base, base + int(lay.k_len[b]))
        scores = O.indexer_scores(qi, w, O.dequant_e4m3(kc, ks), wl.index_scale)
        idx = O.topk_indices(scores, wl.top_k)
        assert set(lay.needle_pos[b].tolist()) <= set(idx.tolist())


def test_drift_shared_within_block():
    s = synth.Synth(synth.WORKLOADS["prefill_64k"])
    d = s._drift(250, 520, 8, 1)
    assert np.array_equal(d[0], d[5])          # rows 250, 255: block 0
    assert np.array_equal(d[6], d[261])        # rows 256, 511: block 1
    assert not np.array_equal(d[5], d[6])


def test_paged_pools_poison_and_map():
    # a small paged workload of the same construction
    wl = synth.Workload("paged_small", 4, "decode", 3, 0, ctx_range=(70, 200), paged=True,
                        h_i=2, d_i=16, top_k=8, heads=2, d_c=8, d_r=8)
    s = synth.Synth(wl)
    lay = s.layout
    ki_pool, ks_pool, kv_pool = s.paged_pools()
    for b in range(wl.batch):
        n = int(lay.k_len[b])
        base = int(lay.k_seq_start[b])
        kc, ks = s.ki(base, base + n)
        kv = s.kv(base, base + n)
        assert np.array_equal(O.unpage(ki_pool, lay.page_table[b], n, 64), kc)
        assert np.array_equal(O.unpage(ks_pool[..., None], lay.page_table[b], n, 64)[:, 0], ks)
        assert np.array_equal(O.unpage(kv_pool, lay.page_table[b], n, 64), kv)
        last = lay.page_table[b, (n - 1) // 64]
        tail = n % 64
        if tail:
            assert (ki_pool[last, tail:] == 0x7F).all() and np.isnan(ks_pool[last, tail:]).all()
            assert (kv_pool[last, tail:] == 0x7FC0).all()


def test_paged_pools_fp32():
    # fp32 workloads: fp32 key and latent pools, no scales, NaN in unused slots
    wl = synth.Workload("paged_small_f32", 5, "decode", 3, 0, ctx_range=(70, 200), paged=True,
                        h_i=2, d_i=16, fp8=False, top_k=8, heads=2, d_c=8, d_r=8)
    s = synth.Synth(wl)
    lay = s.layout
    ki_pool, ks_pool, kv_pool = s.paged_pools()
    assert ks_pool is None and ki_pool.dtype == np.float32 and kv_pool.dtype == np.float32
    for b in range(wl.batch):
        n = int(lay.k_len[b])
        base = int(lay.k_seq_start[b])
        k, none = s.ki(base, base + n)
        assert none is None
        assert np.array_equal(O.unpage(ki_pool, lay.page_table[b], n, 64), k)
        assert np.array_equal(O.unpage(kv_pool, lay.page_table[b], n, 64), s.kv(base, base + n))
        last = lay.page_table[b, (n - 1) // 64]
        tail = n % 64
        if tail:
            assert np.isnan(ki_pool[last, tail:]).all() and np.isnan(kv_pool[last, tail:]).all()
