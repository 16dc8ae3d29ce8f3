"""Decode-step cache append, bit-exact against the oracle: whole key, scale
and latent pools after the HIP kernel writes a batch of new tokens, compared
with the oracle applied to the same pools.  Pools start filled with random
bytes, so a row written where it should not be, or a row left unwritten,
shows up as a mismatch.  Keys include the cases the quantiser branches on:
an all-zero row (scale 1), a single non-zero value, signed zeros, tiny and
huge magnitudes, values near the E4M3 subnormal range."""

import numpy as np
import pytest
import torch

from oracle import cache_oracle as C
from sparse_attention_long_fp8_amd import binding as B

pytestmark = pytest.mark.gpu

PS = 64


def _keys(rng, n, d):
    k = rng.standard_normal((n, d)).astype(np.float32)
    k *= (10.0 ** rng.uniform(-4, 4, (n, 1))).astype(np.float32)
    if n >= 6:
        k[0] = 0.0                                        # all zero: scale 1
        k[1] = 0.0
        k[1, d // 2] = -3.5                               # one value: code -448 there
        k[2] = np.where(rng.random(d) < 0.5, np.float32(-0.0), np.float32(0.0))
        k[2, 0] = 1e-30                                   # the rest underflow to signed zeros
        k[3] *= np.float32(1e-38)                         # subnormal fp32 inputs
        k[4] = rng.integers(-448, 449, d).astype(np.float32) / 448.0 * 2.0 ** -8  # near E4M3 subnormals
    return k


def _pools(rng, rows_shape, d_i, d_c):
    kp = rng.integers(0, 256, rows_shape + (d_i,), dtype=np.uint8)
    sp = rng.standard_normal(rows_shape).astype(np.float32)
    lp = rng.integers(0, 65536, rows_shape + (d_c,), dtype=np.uint16) if d_c else None
    return kp, sp, lp


def _run(gpu, layout_dev, layout_np, seq, pos, k_new, lat_new, kp, sp, lp):
    d_i = k_new.shape[1]
    d_c = 0 if lat_new is None else lat_new.shape[1]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
    kp_d, sp_d = t(kp), t(sp)
    lp_d = None if lp is None else t(lp.view(np.int16))
    B.dsa_cache_append(layout_dev, len(seq), t(seq.astype(np.int32)), t(pos.astype(np.int32)), d_i, t(k_new),
                       kp_d, sp_d, d_c, None if lat_new is None else t(lat_new.view(np.int16)), lp_d)
    torch.cuda.synchronize()
    want = C.cache_append(layout_np, seq, pos, k_new, lat_new, kp, sp, lp)
    assert (kp_d.cpu().numpy() == want[0]).all(), "E4M3 key codes differ"
    got_s = sp_d.cpu().numpy()
    assert (got_s.view(np.uint32) == want[1].view(np.uint32)).all(), "key scales differ"
    if lp is not None:
        assert (lp_d.cpu().numpy().view(np.uint16) == want[2]).all(), "latent rows differ"


def _paged(rng, k_len, gpu):
    pages = [-(-n // PS) for n in k_len]
    P = sum(pages)
    perm = rng.permutation(P).astype(np.int32)
    stride = max(pages)
    table = -np.ones((len(k_len), stride), np.int32)
    c = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[c:c + n]
        c += n
    tab_d = torch.from_numpy(table).to(gpu)
    lay = B.make_paged_layout(tab_d, stride, P, PS)
    return lay, tab_d, {"paged": True, "page_table": table, "page_size": PS}, P


@pytest.mark.parametrize("d_i,d_c", [(128, 576), (32, 0), (512, 8)])
def test_decode_step_append_paged(gpu, d_i, d_c):
    rng = np.random.default_rng(100 + d_i + d_c)
    k_len = rng.integers(1, 700, 37)                      # histories after the step
    lay, _keep, lay_np, P = _paged(rng, k_len, gpu)
    seq = rng.permutation(len(k_len)).astype(np.int32)    # one new token per sequence, any order
    pos = (k_len[seq] - 1).astype(np.int32)               # at the end of its history
    k_new = _keys(rng, len(seq), d_i)
    lat = rng.integers(0, 65536, (len(seq), d_c), dtype=np.uint16) if d_c else None
    kp, sp, lp = _pools(rng, (P, PS), d_i, d_c)
    _run(gpu, lay, lay_np, seq, pos, k_new, lat, kp, sp, lp)


def test_prefill_chunk_append_contiguous(gpu):
    rng = np.random.default_rng(7)
    d_i, d_c = 128, 576
    k_len = np.array([300, 1000, 17], np.int64)
    k_seq_start = np.concatenate([[0], np.cumsum(k_len)]).astype(np.int64)
    N = int(k_seq_start[-1])
    ks_d = torch.from_numpy(k_seq_start).to(gpu)
    lay = B.make_contiguous_layout(ks_d, N)
    # a chunk of sequence 1 (positions 200..899) plus the tail of sequence 0
    seq = np.concatenate([np.full(700, 1), np.full(40, 0)]).astype(np.int32)
    pos = np.concatenate([np.arange(200, 900), np.arange(260, 300)]).astype(np.int32)
    k_new = _keys(rng, len(seq), d_i)
    lat = rng.integers(0, 65536, (len(seq), d_c), dtype=np.uint16)
    kp, sp, lp = _pools(rng, (N,), d_i, d_c)
    _run(gpu, lay, {"k_seq_start": k_seq_start}, seq, pos, k_new, lat, kp, sp, lp)


def test_empty_append_writes_nothing(gpu):
    rng = np.random.default_rng(1)
    lay, _keep, lay_np, P = _paged(rng, [100], gpu)
    kp, sp, lp = _pools(rng, (P, PS), 128, 576)
    _run(gpu, lay, lay_np, np.zeros(0, np.int32), np.zeros(0, np.int32),
         np.zeros((0, 128), np.float32), np.zeros((0, 576), np.uint16), kp, sp, lp)


def test_appended_keys_score_like_the_harness(gpu):
    """An appended key row decodes to what the input harness's quantiser
    stores for the same fp32 row: the indexer reads the same bytes either way."""
    from sparse_attention_long_fp8_amd import synth
    rng = np.random.default_rng(3)
    k_len = [130]
    lay, _keep, lay_np, P = _paged(rng, k_len, gpu)
    k_new = _keys(rng, 130, 128)
    seq = np.zeros(130, np.int32)
    pos = np.arange(130, dtype=np.int32)
    kp = np.zeros((P, PS, 128), np.uint8)
    sp = np.zeros((P, PS), np.float32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
    kp_d, sp_d = t(kp), t(sp)
    B.dsa_cache_append(lay, 130, t(seq), t(pos), 128, t(k_new), kp_d, sp_d)
    torch.cuda.synchronize()
    codes, scales = synth.quantize_e4m3_per_token(k_new)
    table = lay_np["page_table"][0]
    got = kp_d.cpu().numpy()
    got_s = sp_d.cpu().numpy()
    for p in range(130):
        page, slot = table[p // PS], p % PS
        assert (got[page, slot] == codes[p]).all()
        assert got_s[page, slot] == scales[p]
