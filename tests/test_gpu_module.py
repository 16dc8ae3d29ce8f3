"""The page's complete DSA module (dsa_module_forward), fp32, against the
float64 oracle that follows the page's steps (per-token decompression of the
selected keys and values).

Selection: the GPU's indices may differ from the oracle's only at near-ties
of the k-th score (same bar as the main path).  Output: the oracle is run on
the GPU's own indices; every product is fp32 with sums of at most a few
thousand terms, so the error sits near 1e-6 of the output's scale and the bar
is max |out_gpu - out_ref| <= 1e-4 * max |out_ref| per batch element.
Inputs follow the page's verification: N(0, 1) hidden states and latents,
and weights drawn like its linear layers' default initialisation,
U(-1/sqrt(fan_in), 1/sqrt(fan_in))."""

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from oracle import module_oracle as M
from sparse_attention_long_fp8_amd import binding as B

pytestmark = pytest.mark.gpu

TOL = 1e-4
TIE_RTOL = 1e-3


def _lin(rng, out_f, in_f):
    b = 1.0 / np.sqrt(in_f)
    return rng.uniform(-b, b, (out_f, in_f)).astype(np.float32)


@pytest.mark.parametrize("Bn,S,hidden,H,d_h,d_c,d_i,top_k", [
    (2, 16384, 1024, 16, 64, 256, 32, 512),   # the page's verification shape
    (3, 300, 256, 4, 32, 128, 16, 512),       # top_k > history: every key kept, -1 padding
    (1, 2000, 128, 8, 16, 64, 8, 64),
    (6, 700, 256, 4, 32, 128, 16, 100),       # batch > 4: a second pass of every matrix-vector kernel
    (5, 333, 130, 3, 10, 50, 7, 96),          # widths not multiples of 4: the scalar paths throughout
])
def test_module_forward_matches_oracle(gpu, Bn, S, hidden, H, d_h, d_c, d_i, top_k):
    rng = np.random.default_rng(S + H)
    qh = rng.standard_normal((Bn, hidden)).astype(np.float32)
    hist = rng.standard_normal((Bn, S, hidden)).astype(np.float32)
    lat = rng.standard_normal((Bn, S, d_c)).astype(np.float32)
    W = [_lin(rng, d_i, hidden), _lin(rng, d_i, hidden), _lin(rng, H * d_h, hidden), _lin(rng, H * d_h, d_c),
         _lin(rng, H * d_h, d_c), _lin(rng, hidden, H * d_h)]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
    out = torch.full((Bn, hidden), float("nan"), device=gpu)
    idx = torch.full((Bn, top_k), -7, dtype=torch.int32, device=gpu)
    nb = B.dsa_module_forward_workspace_size(Bn, S, hidden, H, d_h, d_c, d_i)
    ws = torch.empty(nb + 256, dtype=torch.uint8, device=gpu)
    base = ws.data_ptr() + (-ws.data_ptr()) % 256
    B.dsa_module_forward(Bn, S, hidden, H, d_h, d_c, d_i, top_k, t(qh), t(hist), t(lat), *[t(w) for w in W],
                         out, idx, base, nb)
    torch.cuda.synchronize()
    got_out, got_idx = out.cpu().numpy().astype(np.float64), idx.cpu().numpy()
    W_qi, W_ki, W_q, W_uk, W_uv, W_out = W
    m = min(top_k, S)
    for b in range(Bn):
        # selection, end to end against the oracle's scores
        scores = np.maximum((hist[b].astype(np.float64) @ W_ki.T.astype(np.float64))
                            @ (W_qi.astype(np.float64) @ qh[b].astype(np.float64)), 0.0) / np.sqrt(d_i)
        want = O.topk_indices(scores, top_k)
        g = got_idx[b]
        assert (g[m:] == -1).all() and (np.diff(g[:m]) > 0).all() and g[:m].min() >= 0 and g[m - 1] < S
        diff = np.setxor1d(g[:m], want[:m])
        if diff.size:
            tau = scores[want[:m]].min()
            assert (np.abs(scores[diff] - tau) <= TIE_RTOL * abs(tau)).all(), "batch %d: selection differs" % b
        # output on the GPU's own selection
        ref = M.attention_given_indices(qh[b], lat[b], g, W_q, W_uk, W_uv, W_out, H, d_h)
        err = np.abs(got_out[b] - ref).max() / np.abs(ref).max()
        assert err <= TOL, "batch %d: relative error %.3g" % (b, err)
