"""Pins for the output-projection oracle: brute-force sums on tiny shapes,
closed forms (selection and identity weights), linearity."""

import numpy as np

from oracle import proj_oracle as P


def test_matches_brute_force_loops():
    rng = np.random.default_rng(0)
    T, H, d_c, d_h, hidden = 3, 2, 5, 3, 4
    o = rng.normal(size=(T, H, d_c))
    w_uv = rng.normal(size=(H * d_h, d_c))
    w_o = rng.normal(size=(hidden, H * d_h))
    out, y = P.output_projection(o, w_uv, w_o, d_h)
    for t in range(T):
        for h in range(H):
            for d in range(d_h):
                want = sum(w_uv[h * d_h + d, c] * o[t, h, c] for c in range(d_c))
                assert abs(y[t, h, d] - want) < 1e-12
        for j in range(hidden):
            want = sum(w_o[j, h * d_h + d] * y[t, h, d] for h in range(H) for d in range(d_h))
            assert abs(out[t, j] - want) < 1e-12


def test_selection_and_identity_weights():
    rng = np.random.default_rng(1)
    T, H, d_c, d_h = 4, 3, 8, 2
    o = rng.normal(size=(T, H, d_c))
    w_uv = np.zeros((H * d_h, d_c))
    for h in range(H):
        w_uv[h * d_h:(h + 1) * d_h, :d_h] = np.eye(d_h)   # W_UV,h picks latent dims 0..d_h-1
    out, _ = P.output_projection(o, w_uv, np.eye(H * d_h), d_h)
    assert np.array_equal(out, o[:, :, :d_h].reshape(T, H * d_h))


def test_linear_in_the_input_and_permutes_with_output_rows():
    rng = np.random.default_rng(2)
    T, H, d_c, d_h, hidden = 5, 2, 6, 3, 7
    o = rng.normal(size=(T, H, d_c))
    w_uv = rng.normal(size=(H * d_h, d_c))
    w_o = rng.normal(size=(hidden, H * d_h))
    out, _ = P.output_projection(o, w_uv, w_o, d_h)
    out2, _ = P.output_projection(2.0 * o, w_uv, w_o, d_h)
    assert np.array_equal(out2, 2.0 * out)
    perm = rng.permutation(hidden)
    out3, _ = P.output_projection(o, w_uv, w_o[perm], d_h)
    assert np.array_equal(out3, out[:, perm])
