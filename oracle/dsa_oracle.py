"""Plain CPU oracle for the DeepSeek Sparse Attention (DSA) hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test-suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library (no
kernels, headers, tables or helpers); the two meet only through the seeded
input generator, which holds none of the method's arithmetic.

Everything here is float64 numpy, written to be read against the pages, not to
be fast.  Library primitives used as single steps: ``@`` (matmul), ``np.exp``,
``np.log``, ``np.lexsort`` and ``np.sort``.  There is no blocking, fusion or
reordering beyond the definitions cited on each function.

Sources (page title, then section / equation):
  [DSA-guide] "DeepSeek Sparse Attention DSA Architecture Guide"
      - "Stage 1: The Lightning Indexer", equation for I_{t,s} (ReLU score),
        and its item 3 (per-key separable scores, top-k commutes over tiles)
      - "Stage 2: Fine-Grained Token Selection", equations for S_t (TopK),
        C_t / K_t^R (gather) and u_{t,i} (softmax restricted to S_t)
      - "The Classical Multi-Head Latent Attention (MLA) Mechanism", equation
        for A_{t,s,i} (latent + decoupled rotary logit over sqrt(d_h + d_R))
      - "End-to-End Implementation" code: k = min(top_k, seq_len), selected
        positions re-sorted ascending to keep temporal order
  [paged] "Sparse Attention in Large Language Models: Architecture Evolution
      and Engineering Practice", section 4.1 (paged KV-cache management)

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):
  * indexer: the multi-head weighted form I = scale * sum_j w_j ReLU(q_j . k);
    the pages' single-head form is H_I = 1, w = 1, scale = 1/sqrt(d_I);
  * FP8 is OCP E4M3 (bias 7, no infinities, 0x7F / 0xFF = NaN, max 448) with
    one fp32 scale per query token (shared by its heads) and per key token;
  * causal, self-inclusive: query at position p sees keys 0..p (n = p + 1);
  * top-k keeps m = min(k, n) positions, ties broken toward the lowest
    position, written ascending and padded with -1;
  * MLA is in absorbed (MQA) form: one key row of width D_qk per token shared
    by all heads, the value is its first D_v entries, the softmax scale is an
    explicit argument; output stays in latent space.

Parity pins: every function below is pinned by tests that do not call this
module's arithmetic twice (brute force, closed forms, library routines,
hand-derived fixtures).  See tests/test_oracle.py.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "E4M3_TABLE",
    "decode_e4m3",
    "decode_bf16",
    "dequant_e4m3",
    "query_rows",
    "unpage",
    "indexer_scores",
    "topk_indices",
    "sparse_mla",
    "dense_causal_mla",
    "forward_row",
]


# --------------------------------------------------------------------------
# O-1  number formats
# --------------------------------------------------------------------------
def _build_e4m3_table() -> np.ndarray:
    """Value of every OCP FP8 E4M3 byte, as float64.

    Sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.  Exponent
    field 0 is subnormal: (m/8) * 2^-6.  Otherwise (1 + m/8) * 2^(e-7).
    S.1111.111 is NaN; the format has no infinities, so S.1111.110 = 448 is
    the largest finite magnitude.  The pages only say "FP8" ([DSA-guide],
    Stage 1, item 1); the encoding is the OCP standard's.
    """
    table = np.empty(256, dtype=np.float64)
    for byte in range(256):
        sign = -1.0 if (byte >> 7) & 1 else 1.0
        e = (byte >> 3) & 0xF
        m = byte & 0x7
        if e == 0xF and m == 0x7:
            table[byte] = np.nan
        elif e == 0:
            table[byte] = sign * (m / 8.0) * 2.0 ** -6
        else:
            table[byte] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return table


E4M3_TABLE = _build_e4m3_table()


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """uint8 E4M3 codes -> float64 values (exact)."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("E4M3 codes must be uint8")
    return E4M3_TABLE[codes]


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64 values (exact).

    A bfloat16 is the upper half of an IEEE binary32, so widening is a
    16-bit left shift of the pattern.
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("bfloat16 values must be given as uint16 bit patterns")
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequant_e4m3(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Per-token dequantisation: value = decode(code) * scale[token].

    ``codes`` has the token axis first; ``scale`` holds one fp32 per token.
    The product of a 4-bit-mantissa value and a 24-bit-mantissa scale is
    exact in float64.
    """
    vals = decode_e4m3(codes)
    sc = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return vals * sc.reshape(sc.shape + (1,) * (vals.ndim - sc.ndim))


# --------------------------------------------------------------------------
# batch bookkeeping
# --------------------------------------------------------------------------
def query_rows(q_seq_start, k_len):
    """For each query row: (sequence b, position p, candidates n = p + 1).

    Sequence b owns query rows q_seq_start[b] .. q_seq_start[b+1]-1 and a key
    history of k_len[b] tokens.  Its nq queries are the last nq tokens of that
    history, so query i sits at p = k_len[b] - nq + i and, causally and
    self-inclusively, sees keys 0..p ([DSA-guide] Stage 1: "s <= t").
    """
    q_seq_start = [int(x) for x in q_seq_start]
    k_len = [int(x) for x in k_len]
    rows = []
    for b in range(len(k_len)):
        nq = q_seq_start[b + 1] - q_seq_start[b]
        if nq < 0 or nq > k_len[b]:
            raise ValueError("sequence %d: %d queries but %d keys" % (b, nq, k_len[b]))
        for i in range(nq):
            p = k_len[b] - nq + i
            rows.append((b, p, p + 1))
    return rows


def unpage(pool: np.ndarray, page_table_row, n: int, page_size: int) -> np.ndarray:
    """Logical rows 0..n-1 of one sequence from a paged pool.

    Logical position s lives in physical page page_table_row[s // page_size]
    at slot s % page_size ([paged] section 4.1 recommends paged KV storage).
    """
    out = []
    for s in range(n):
        page = int(page_table_row[s // page_size])
        if page < 0:
            raise ValueError("position %d maps to an unassigned page" % s)
        out.append(pool[page, s % page_size])
    if not out:
        return pool[:0, 0]
    return np.stack(out)


# --------------------------------------------------------------------------
# O-2  lightning-indexer scores
# --------------------------------------------------------------------------
def indexer_scores(q_t: np.ndarray, w_t: np.ndarray, keys: np.ndarray,
                   scale: float = 1.0) -> np.ndarray:
    """Indexer scores of one query row against keys 0..n-1.

    I[s] = scale * sum_j w[j] * ReLU( sum_d q[j, d] * k[s, d] )

    [DSA-guide] Stage 1 gives the single-head score ReLU(q.k / sqrt(d_I));
    this is its multi-head weighted form.  ReLU is applied per head, before
    the head weight.  q_t: [H_I, d_I], w_t: [H_I], keys: [n, d_I]; all
    already dequantised to float64.  Returns float64 [n].
    """
    q_t = np.asarray(q_t, dtype=np.float64)
    w_t = np.asarray(w_t, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    dots = keys @ q_t.T                       # [n, H_I]: q_j . k_s
    relu = np.maximum(dots, 0.0)              # ReLU per head
    return float(scale) * (relu @ w_t)        # weighted sum over heads


# --------------------------------------------------------------------------
# O-3  top-k selection
# --------------------------------------------------------------------------
def topk_indices(scores: np.ndarray, k: int) -> np.ndarray:
    """Positions of the min(k, n) largest scores, ascending, -1 padded.

    [DSA-guide] Stage 2: S_t = TopK({I_{t,s}}_{s<=t}, k); its implementation
    uses k = min(top_k, seq_len) and re-sorts the chosen positions ascending.
    Ties go to the lowest position.  Scores compare by value (-0 == +0);
    a NaN score is a precondition violation.
    """
    scores = np.asarray(scores, dtype=np.float64)
    if np.isnan(scores).any():
        raise ValueError("NaN score: top-k is undefined")
    n = scores.shape[0]
    m = min(int(k), n)
    positions = np.arange(n)
    # np.lexsort: last key is primary.  Primary: larger score first;
    # secondary: lower position first.
    order = np.lexsort((positions, -scores))
    chosen = np.sort(order[:m])
    out = np.full(int(k), -1, dtype=np.int64)
    out[:m] = chosen
    return out


# --------------------------------------------------------------------------
# O-4  sparse MLA (absorbed / MQA form)
# --------------------------------------------------------------------------
def sparse_mla(q_t: np.ndarray, kv: np.ndarray, idx: np.ndarray, d_v: int,
               sm_scale: float):
    """Attention of one query row over the selected key rows.

    For each head h, with J the selected positions (idx != -1):
        z_j   = sm_scale * q[h, :] . kv[s_j, :]         (D_qk-wide)
        p_j   = exp(z_j - max z) / sum_j exp(z_j - max z)
        o[h]  = sum_j p_j * kv[s_j, :d_v]
        lse   = max z + log sum_j exp(z_j - max z)

    [DSA-guide] Stage 2 (gather of c^KV and k^R for s in S_t; u_t with the
    softmax taken over S_t only) and the MLA logit of the classical MLA
    section ([c_s ; k^R_s] is one key row, so the rotary part is the tail of
    the row).  Output stays in latent space (before W_UV).  An empty
    selection gives o = 0 and lse = -inf.
    q_t: [H, D_qk]; kv: [n, D_qk] logical rows of this sequence.
    """
    q_t = np.asarray(q_t, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    idx = np.asarray(idx)
    sel = idx[idx >= 0]
    h = q_t.shape[0]
    if sel.size == 0:
        return np.zeros((h, d_v)), np.full(h, -np.inf)
    rows = kv[sel]                                  # gather: [m, D_qk]
    z = float(sm_scale) * (q_t @ rows.T)            # [H, m]
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    denom = e.sum(axis=1, keepdims=True)
    p = e / denom
    if not np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12):
        raise AssertionError("softmax rows do not sum to one")
    o = p @ rows[:, :d_v]                           # [H, d_v]
    lse = zmax[:, 0] + np.log(denom[:, 0])
    return o, lse


def dense_causal_mla(q: np.ndarray, kv: np.ndarray, d_v: int, sm_scale: float):
    """Dense causal MLA over one sequence: query t attends to every s <= t.

    The classical (non-sparse) attention of [DSA-guide]'s MLA section, for
    checking that selection with k >= t + 1 reduces to it.  Written as a
    plain per-row loop with its own softmax (no max shift needed at the
    sizes it is used for; float64 exp does not overflow there).
    q: [T, H, D_qk]; kv: [T, D_qk].  Returns o [T, H, d_v], lse [T, H].
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    t_len, h, _ = q.shape
    o = np.zeros((t_len, h, d_v))
    lse = np.zeros((t_len, h))
    for t in range(t_len):
        for head in range(h):
            weights = []
            for s in range(t + 1):
                weights.append(np.exp(sm_scale * float(np.dot(q[t, head], kv[s]))))
            total = sum(weights)
            acc = np.zeros(d_v)
            for s in range(t + 1):
                acc += (weights[s] / total) * kv[s, :d_v]
            o[t, head] = acc
            lse[t, head] = np.log(total)
    return o, lse


# --------------------------------------------------------------------------
# the whole path for one query row
# --------------------------------------------------------------------------
def forward_row(qi_t, w_t, keys_i, q_t, kv, n: int, k: int, scale: float,
                d_v: int, sm_scale: float):
    """Indexer -> top-k -> sparse MLA for one query row with n candidates.

    The order of the pipeline figure of [DSA-guide] (indexer scores, top-k
    positions, selective fetch, sparse MLA).  keys_i / kv are the logical
    rows of the query's sequence (at least n of them).
    Returns (scores [n], idx [k], o [H, d_v], lse [H]).
    """
    scores = indexer_scores(qi_t, w_t, np.asarray(keys_i)[:n], scale)
    idx = topk_indices(scores, k)
    o, lse = sparse_mla(q_t, np.asarray(kv)[:n], idx, d_v, sm_scale)
    return scores, idx, o, lse
