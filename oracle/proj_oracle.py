"""Plain CPU oracle for the output projections after sparse MLA.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test-suite and the benchmark's CPU leg use it.
It shares no code with the HIP library.

What it computes ("DeepSeek Sparse Attention DSA Architecture Guide", "Stage
2: Fine-Grained Token Selection", the u_t equation; the implementation
section's w_uv and w_out projections): the sparse stage's per-head output
stays in the compressed latent space, o[t, h] in R^{d_c}; head h's value
up-projection W_UV,h (d_h x d_c) maps it to the head dimension, the heads
are concatenated, and the output projection W_O (hidden x H*d_h) maps the
concatenation to the model width:

    y[t, h, :] = W_UV,h . o[t, h, :]
    out[t, :]  = W_O . concat_h y[t, h, :]

Weights use the page's linear-layer layout (out_features x in_features): the
value up-projection of all heads is one [H*d_h, d_c] matrix whose rows
h*d_h .. h*d_h + d_h - 1 are W_UV,h.  Everything is float64; a matrix product
is a single library step.
"""

from __future__ import annotations

import numpy as np

__all__ = ["output_projection"]


def output_projection(o: np.ndarray, w_uv: np.ndarray, w_o: np.ndarray, d_h: int):
    """o [T, H, d_c], w_uv [H*d_h, d_c], w_o [hidden, H*d_h] -> (out [T, hidden], y [T, H, d_h])."""
    o = np.asarray(o, dtype=np.float64)
    T, H, d_c = o.shape
    w_uv = np.asarray(w_uv, dtype=np.float64).reshape(H, d_h, d_c)
    w_o = np.asarray(w_o, dtype=np.float64)
    y = np.empty((T, H, d_h), dtype=np.float64)
    for h in range(H):
        y[:, h, :] = o[:, h, :] @ w_uv[h].T
    out = y.reshape(T, H * d_h) @ w_o.T
    return out, y
