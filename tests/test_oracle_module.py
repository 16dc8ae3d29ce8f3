"""Pins for the page-module oracle: brute-force loops on a tiny shape, the
absorbed form (W_UK folded into the query, W_UV after the softmax) as an
independent formula, and a uniform softmax closed form."""

import numpy as np

from oracle import module_oracle as M


def _weights(rng, hidden, d_i, heads, d_h, d_c):
    return (rng.normal(size=(d_i, hidden)), rng.normal(size=(d_i, hidden)), rng.normal(size=(heads * d_h, hidden)),
            rng.normal(size=(heads * d_h, d_c)), rng.normal(size=(heads * d_h, d_c)),
            rng.normal(size=(hidden, heads * d_h)))


def test_brute_force_tiny():
    rng = np.random.default_rng(0)
    B, S, hidden, d_i, H, d_h, d_c, k = 1, 6, 5, 2, 2, 3, 4, 3
    W = _weights(rng, hidden, d_i, H, d_h, d_c)
    qh, hist, lat = rng.normal(size=(B, hidden)), rng.normal(size=(B, S, hidden)), rng.normal(size=(B, S, d_c))
    out, idx = M.module_forward(qh, hist, lat, *W, k, H, d_h)
    W_qi, W_ki, W_q, W_uk, W_uv, W_out = W
    sc = []
    for s in range(S):
        dot = sum(sum(W_qi[a, x] * qh[0, x] for x in range(hidden)) * sum(W_ki[a, x] * hist[0, s, x]
                  for x in range(hidden)) for a in range(d_i))
        sc.append(max(dot, 0.0) / np.sqrt(d_i))
    order = sorted(range(S), key=lambda s: (-sc[s], s))[:k]
    assert list(idx[0]) == sorted(order)
    o = []
    for h in range(H):
        q = [sum(W_q[h * d_h + d, x] * qh[0, x] for x in range(hidden)) for d in range(d_h)]
        logits, vals = [], []
        for s in sorted(order):
            Kv = [sum(W_uk[h * d_h + d, c] * lat[0, s, c] for c in range(d_c)) for d in range(d_h)]
            Vv = [sum(W_uv[h * d_h + d, c] * lat[0, s, c] for c in range(d_c)) for d in range(d_h)]
            logits.append(sum(q[d] * Kv[d] for d in range(d_h)) / np.sqrt(d_h))
            vals.append(Vv)
        mx = max(logits)
        e = [np.exp(z - mx) for z in logits]
        o.extend(sum(e[j] * vals[j][d] for j in range(len(e))) / sum(e) for d in range(d_h))
    want = [sum(W_out[r, j] * o[j] for j in range(H * d_h)) for r in range(hidden)]
    assert np.allclose(out[0], want, rtol=1e-12, atol=1e-12)


def test_absorbed_form_is_the_same_function():
    rng = np.random.default_rng(1)
    B, S, hidden, d_i, H, d_h, d_c, k = 2, 40, 16, 4, 3, 5, 8, 12
    W = _weights(rng, hidden, d_i, H, d_h, d_c)
    W_qi, W_ki, W_q, W_uk, W_uv, W_out = W
    qh, hist, lat = rng.normal(size=(B, hidden)), rng.normal(size=(B, S, hidden)), rng.normal(size=(B, S, d_c))
    out, idx = M.module_forward(qh, hist, lat, *W, k, H, d_h)
    for b in range(B):
        c = lat[b][idx[b]]
        q = (W_q @ qh[b]).reshape(H, d_h)
        o = []
        for h in range(H):
            q_abs = W_uk[h * d_h:(h + 1) * d_h].T @ q[h]          # fold W_UK into the query
            z = c @ q_abs / np.sqrt(d_h)
            a = np.exp(z - z.max())
            a /= a.sum()
            o.append(W_uv[h * d_h:(h + 1) * d_h] @ (a @ c))         # W_UV after the softmax
        assert np.allclose(out[b], W_out @ np.concatenate(o), rtol=1e-10, atol=1e-10)


def test_uniform_softmax_is_the_mean_of_the_values():
    rng = np.random.default_rng(2)
    S, hidden, H, d_h, d_c = 30, 8, 2, 4, 6
    W = list(_weights(rng, hidden, 3, H, d_h, d_c))
    W[2] = np.zeros_like(W[2])                                     # q = 0: every logit 0
    lat = rng.normal(size=(1, S, d_c))
    idx = np.array([1, 4, 9, 22, -1, -1])
    out = M.attention_given_indices(rng.normal(size=hidden), lat[0], idx, W[2], W[3], W[4], W[5], H, d_h)
    v = (lat[0][[1, 4, 9, 22]] @ W[4].T).mean(axis=0)
    assert np.allclose(out, W[5] @ v, rtol=1e-12, atol=1e-12)
