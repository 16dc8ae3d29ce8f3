"""Pins for the cache-append oracle (oracle/cache_oracle.py): its E4M3
encoder against torch's float8_e4m3fn cast (a library routine), closed-form
rows, the input harness's independent quantiser, and paged vs contiguous
addressing."""

import numpy as np
import pytest
import torch

from oracle import cache_oracle as C
from oracle import dsa_oracle as O
from sparse_attention_long_fp8_amd import synth


def _torch_e4m3(y):
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = O.decode_e4m3(codes).astype(np.float32)
    got = C.encode_e4m3_rne(vals)
    # +0 and -0 both survive with their sign bit
    assert (got == codes).all()


def test_encode_ties_go_to_the_even_code():
    # exact midpoints between consecutive finite magnitudes (representable in fp32)
    v = O.E4M3_TABLE[:0x7F]
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    assert (mids.astype(np.float64) == (v[:-1] + v[1:]) / 2).all()
    got = C.encode_e4m3_rne(mids)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert (got == want).all()
    assert (C.encode_e4m3_rne(-mids) == (want | 0x80)).all()
    assert (got == _torch_e4m3(mids)).all()


def test_encode_matches_torch_cast_on_random_values():
    rng = np.random.default_rng(11)
    y = np.concatenate([
        rng.uniform(-448, 448, 200000),
        rng.normal(0, 1, 100000),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 100000),  # subnormal range
        np.array([0.0, -0.0, 448.0, -448.0, 2.0 ** -10, -2.0 ** -10, 2.0 ** -9, 3 * 2.0 ** -10]),
    ]).astype(np.float32)
    assert (C.encode_e4m3_rne(y) == _torch_e4m3(y)).all()


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        C.encode_e4m3_rne(np.array([448.5], np.float32))


def test_quantize_token_closed_forms():
    # the largest magnitude maps to +-448 exactly, whatever the row
    x = np.array([0.5, -3.0, 1.25, 2.0], np.float32)
    codes, scale = C.quantize_token(x)
    assert scale == np.float32(3.0) / np.float32(448.0)
    assert codes[1] == 0xFE
    # all-zero row: scale 1, all codes +0
    codes, scale = C.quantize_token(np.zeros(128, np.float32))
    assert scale == 1.0 and (codes == 0).all()
    # a row of one repeated value: every code is 448
    codes, scale = C.quantize_token(np.full(64, -7.0, np.float32))
    assert (codes == 0xFE).all() and scale == np.float32(7.0) / np.float32(448.0)
    # dequantised error within half a code step of the scaled value
    rng = np.random.default_rng(3)
    x = rng.normal(size=128).astype(np.float32)
    codes, scale = C.quantize_token(x)
    back = O.decode_e4m3(codes) * np.float64(scale)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -4 + np.float64(scale) * 2.0 ** -10)


def test_quantize_token_matches_the_input_harness():
    # synth's per-token quantiser casts with torch; the oracle searches the table
    rng = np.random.default_rng(5)
    x = rng.normal(size=(300, 128)).astype(np.float32) * rng.uniform(0.01, 100, (300, 1)).astype(np.float32)
    x[7] = 0.0
    want_codes, want_scale = synth.quantize_e4m3_per_token(x)
    for i in range(x.shape[0]):
        codes, scale = C.quantize_token(x[i])
        assert scale == want_scale[i]
        assert (codes == want_codes[i]).all()


def test_append_paged_equals_contiguous():
    rng = np.random.default_rng(9)
    B, ps, d, dc = 3, 64, 32, 16
    k_len = [70, 5, 130]
    k_seq_start = np.concatenate([[0], np.cumsum(k_len)])
    pages = [-(-n // ps) for n in k_len]
    perm = rng.permutation(sum(pages))
    table = -np.ones((B, 4), np.int32)
    c = 0
    for b in range(B):
        table[b, :pages[b]] = perm[c:c + pages[b]]
        c += pages[b]
    seq = np.array([0, 2, 1, 2], np.int32)
    pos = np.array([69, 129, 4, 64], np.int32)
    k_new = rng.normal(size=(4, d)).astype(np.float32)
    lat = rng.integers(0, 0x7F00, size=(4, dc)).astype(np.uint16)
    N = int(k_seq_start[-1])
    kc, sc, lc = C.cache_append({"k_seq_start": k_seq_start}, seq, pos, k_new, lat,
                                np.zeros((N, d), np.uint8), np.zeros(N, np.float32), np.zeros((N, dc), np.uint16))
    P = sum(pages)
    kp, sp, lp = C.cache_append({"paged": True, "page_table": table, "page_size": ps}, seq, pos, k_new, lat,
                                np.zeros((P, ps, d), np.uint8), np.zeros((P, ps), np.float32),
                                np.zeros((P, ps, dc), np.uint16))
    for b in range(B):
        rows = slice(int(k_seq_start[b]), int(k_seq_start[b + 1]))
        assert (O.unpage(kp, table[b], k_len[b], ps) == kc[rows]).all()
        assert (O.unpage(sp[..., None], table[b], k_len[b], ps)[:, 0] == sc[rows]).all()
        assert (O.unpage(lp, table[b], k_len[b], ps) == lc[rows]).all()
    # exactly the four addressed rows changed
    assert int((sc != 0).sum()) == 4
