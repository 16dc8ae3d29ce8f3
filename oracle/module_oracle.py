"""Plain CPU oracle for the page's complete DSA module (non-absorbed form).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test-suite and the benchmark's CPU leg use it.
It shares no code with the HIP library.

What it computes: the module of "DeepSeek Sparse Attention DSA Architecture
Guide", section "End-to-End Implementation" (its DeepSeekSparseAttention and
LightningIndexer classes), for one query token per batch element over a
history of S tokens, in the order the page computes it:
  1. indexer: q_I = W_qI h_q, k_I[s] = W_kI h_s, I[s] = ReLU(q_I . k_I[s]) / sqrt(d_I)
     (the page scales before the ReLU; the scale is positive, so the order
     does not matter);
  2. m = min(top_k, S) positions with the largest I, ascending; ties go to
     the lowest position (the page's topk leaves them open);
  3. the selected latent rows c_s are decompressed per token into keys and
     values, K = W_UK c_s and V = W_UV c_s, one d_h-vector per head;
  4. per head, softmax over the selected tokens of (q_h . K_h) / sqrt(d_h),
     q = W_Q h_q, and the weighted sum of V_h;
  5. out = W_out concat_h o_h.
Weights are in the page's linear-layer layout [out_features, in_features].
Everything is float64; matrix products, np.exp and the oracle's top-k are
single steps.
"""

from __future__ import annotations

import numpy as np

from .dsa_oracle import topk_indices

__all__ = ["module_forward", "attention_given_indices"]


def attention_given_indices(q_hidden_b, latent_b, idx, W_q, W_uk, W_uv, W_out, heads, head_dim):
    """Steps 3-5 for one batch element on a given selection (positions >= 0)."""
    sel = np.asarray(latent_b, dtype=np.float64)[np.asarray(idx)[np.asarray(idx) >= 0]]
    K = (sel @ np.asarray(W_uk, np.float64).T).reshape(len(sel), heads, head_dim)
    V = (sel @ np.asarray(W_uv, np.float64).T).reshape(len(sel), heads, head_dim)
    q = (np.asarray(W_q, np.float64) @ np.asarray(q_hidden_b, np.float64)).reshape(heads, head_dim)
    o = np.empty((heads, head_dim))
    for h in range(heads):
        z = K[:, h, :] @ q[h] / np.sqrt(head_dim)
        e = np.exp(z - z.max())
        a = e / e.sum()
        o[h] = a @ V[:, h, :]
    return np.asarray(W_out, np.float64) @ o.reshape(heads * head_dim)


def module_forward(q_hidden, hist, latent, W_qi, W_ki, W_q, W_uk, W_uv, W_out, top_k, heads, head_dim):
    """q_hidden [B, hidden], hist [B, S, hidden], latent [B, S, d_c] -> (out [B, hidden], idx [B, top_k])."""
    q_hidden = np.asarray(q_hidden, np.float64)
    B, S = hist.shape[0], hist.shape[1]
    d_i = W_qi.shape[0]
    out = np.empty((B, W_out.shape[0]))
    idx_all = -np.ones((B, top_k), dtype=np.int64)
    for b in range(B):
        q_i = np.asarray(W_qi, np.float64) @ q_hidden[b]
        k_i = np.asarray(hist[b], np.float64) @ np.asarray(W_ki, np.float64).T
        scores = np.maximum(k_i @ q_i, 0.0) / np.sqrt(d_i)
        idx = topk_indices(scores, top_k)
        idx_all[b] = idx
        out[b] = attention_given_indices(q_hidden[b], latent[b], idx, W_q, W_uk, W_uv, W_out, heads, head_dim)
    return out, idx_all
