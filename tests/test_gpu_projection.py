"""Output projections (dsa_output_projection) against the float64 oracle.

Tolerance: the GEMMs accumulate in fp32, but the intermediate y and the
output are rounded to bf16 (relative error <= 2^-9 each); over sums of random
sign the output's error stays a few 2^-9 of its scale, so the bar is
max |out_gpu - out_ref| <= 1e-2 * max |out_ref| per row (the attention bar)."""

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from oracle import proj_oracle as P
from sparse_attention_long_fp8_amd import binding as B
from sparse_attention_long_fp8_amd import synth

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module")
def blaslt(gpu):
    h = B.dsa_blaslt_create()
    yield h
    B.dsa_blaslt_destroy(h)


def _bf16_dev(x, dev):
    bits = synth.to_bf16_bits(x)
    return bits, torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)


@pytest.mark.parametrize("T,heads,d_c,d_h,hidden", [(37, 128, 512, 128, 7168), (300, 128, 512, 128, 7168),
                                                     (5, 4, 64, 16, 40)])
def test_projection_matches_oracle(gpu, blaslt, T, heads, d_c, d_h, hidden):
    rng = np.random.default_rng(T + heads)
    o_bits, o = _bf16_dev(rng.standard_normal((T, heads, d_c)).astype(np.float32), gpu)
    wuv_bits, w_uv = _bf16_dev((rng.standard_normal((heads * d_h, d_c)) / np.sqrt(d_c)).astype(np.float32), gpu)
    wo_bits, w_o = _bf16_dev((rng.standard_normal((hidden, heads * d_h)) / np.sqrt(heads * d_h)).astype(np.float32),
                             gpu)
    out = torch.full((T, hidden), float("nan"), dtype=torch.bfloat16, device=gpu)
    nb = B.dsa_output_projection_workspace_size(T, heads, d_h)
    ws = torch.empty(nb + 256, dtype=torch.uint8, device=gpu)
    base = ws.data_ptr() + (-ws.data_ptr()) % 256
    B.dsa_output_projection(blaslt, T, heads, d_c, d_h, hidden, o, w_uv, w_o, out, base, nb)
    torch.cuda.synchronize()
    got = O.decode_bf16(out.view(torch.int16).cpu().numpy().view(np.uint16))
    ref, _ = P.output_projection(O.decode_bf16(o_bits), O.decode_bf16(wuv_bits), O.decode_bf16(wo_bits), d_h)
    err = np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)
    assert not np.isnan(got).any()
    assert err.max() <= TOL, "worst row %d: %.3g" % (int(err.argmax()), err.max())


def test_projection_argument_errors(gpu, blaslt):
    nb = B.dsa_output_projection_workspace_size(4, 8, 16)
    assert B.dsa_output_projection(blaslt, 4, 8, 64, 16, 40, 1, 1, 1, 1, 256, nb - 1,
                                   check=False) == B.DSA_ERR_WORKSPACE_TOO_SMALL
    assert B.dsa_output_projection(blaslt, 4, 8, 60, 16, 40, 1, 1, 1, 1, 256, nb, check=False) == B.DSA_ERR_UNSUPPORTED
    assert B.dsa_output_projection(None, 4, 8, 64, 16, 40, 1, 1, 1, 1, 256, nb,
                                   check=False) == B.DSA_ERR_INVALID_ARGUMENT
