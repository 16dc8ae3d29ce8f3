"""Shared machinery of the GPU parity tests: upload one workload's seeded
inputs, run each stage of the HIP path through the C ABI, and compare with
the CPU oracle on the same inputs, to the stated tolerances."""

from __future__ import annotations

import numpy as np
import torch

from oracle import dsa_oracle as O
from sparse_attention_long_fp8_amd import binding as B
from sparse_attention_long_fp8_amd import synth

# Tolerances (stated bars):
#   indexer  |I_gpu - I_ref| <= 1e-3 |I_ref| + 1e-6 max_s |I_ref[t, :]|
#   top-k    bit-exact on identical score arrays; end to end, indices may
#            differ only where the oracle score is within 1e-3 (relative) of
#            the oracle's k-th score
#   attention max |o_gpu - o_ref| / max |o_ref| <= 2e-2 (bf16 inputs), with
#            the oracle run on the GPU's own indices; |lse_gpu - lse_ref| <= 1e-2
IDX_RTOL, IDX_FLOOR = 1e-3, 1e-6
TIE_RTOL = 1e-3
ATTN_TOL_BF16, LSE_TOL = 2e-2, 1e-2
# fp32 inputs: every step is fp32 arithmetic over <= 128-term sums, so the
# error sits near 1e-6 relative; 1e-4 leaves two orders of margin.
ATTN_TOL_F32 = 1e-4


def _i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def _bf16(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def round_up(x, a):
    return (x + a - 1) // a * a


class GpuCase:
    """A workload's inputs on the GPU and, for the oracle, decoded to float64."""

    def __init__(self, wl: synth.Workload, dev, force_contiguous=False):
        self.wl = wl
        self.dev = dev
        s = self.synth = synth.Synth(wl)
        lay = self.lay = s.layout
        self.T = T = lay.num_queries
        self.N = N = int(lay.k_seq_start[-1])
        self.rows = O.query_rows(lay.q_seq_start, lay.k_len)
        self.q_seq_start = _i32(lay.q_seq_start, dev)
        self.k_len = _i32(lay.k_len, dev)
        self.k_seq_start = torch.from_numpy(lay.k_seq_start[:-1].astype(np.int64)).to(dev)
        self.batch = B.make_batch(self.q_seq_start, self.k_len, wl.batch, T, lay.max_q_per_seq, lay.max_k_len)
        self.ld = round_up(lay.max_k_len, 4)

        qi, qs = s.qi(0, T)
        w = s.w(0, T)
        q = s.q(0, T)
        ki, ks = s.ki(0, N)
        kv = s.kv(0, N)
        # oracle side (float64, logical contiguous rows)
        if wl.fp8:
            self.qi_hat = O.dequant_e4m3(qi, qs)
            self.ki_hat = O.dequant_e4m3(ki, ks)
            self.q_hat = O.decode_bf16(q)
            self.kv_hat = O.decode_bf16(kv)
        else:
            self.qi_hat, self.ki_hat = qi.astype(np.float64), ki.astype(np.float64)
            self.q_hat, self.kv_hat = q.astype(np.float64), kv.astype(np.float64)
        self.w_host = w.astype(np.float64)
        # device side
        self.w = torch.from_numpy(w).to(dev)
        self.paged = wl.paged and not force_contiguous
        if wl.fp8:
            self.index_dtype, self.mla_dtype = B.DSA_FP8_E4M3, B.DSA_BF16
            self.qi = torch.from_numpy(qi).to(dev)
            self.qs = torch.from_numpy(qs).to(dev)
            self.q = _bf16(q, dev)
        else:
            self.index_dtype, self.mla_dtype = B.DSA_F32, B.DSA_F32
            self.qi = torch.from_numpy(qi).to(dev)
            self.qs = None
            self.q = torch.from_numpy(q).to(dev)
        if self.paged:
            ki_pool, ks_pool, kv_pool = s.paged_pools()
            self.ki = torch.from_numpy(ki_pool).to(dev)
            self.ks = torch.from_numpy(ks_pool).to(dev) if ks_pool is not None else None
            self.kv = _bf16(kv_pool, dev) if wl.fp8 else torch.from_numpy(kv_pool).to(dev)
            self.page_table = _i32(lay.page_table, dev)
            self.layout = B.make_paged_layout(self.page_table, lay.page_table.shape[1], lay.num_pages)
        else:
            self.ki = torch.from_numpy(ki).to(dev)
            self.ks = torch.from_numpy(ks).to(dev) if wl.fp8 else None
            self.kv = _bf16(kv, dev) if wl.fp8 else torch.from_numpy(kv).to(dev)
            self.layout = B.make_contiguous_layout(self.k_seq_start, max(N, 1))

    # ---------------- GPU path, stage by stage ----------------
    def indexer(self, ld=None):
        ld = ld or self.ld
        scores = torch.full((self.T, ld), float("nan"), device=self.dev)
        wl = self.wl
        B.dsa_indexer_scores(self.batch, self.layout, self.index_dtype, wl.h_i, wl.d_i, self.qi, self.qs, self.w,
                             self.ki, self.ks, wl.index_scale, scores, ld)
        return scores

    def topk(self, scores, ld=None, k=None):
        k = k or self.wl.top_k
        idx = torch.full((self.T, k), -7, dtype=torch.int32, device=self.dev)
        nb = B.dsa_topk_workspace_size(self.batch, k)
        ws = torch.empty(nb + 256, dtype=torch.uint8, device=self.dev) if nb else None
        base = ws.data_ptr() + (-ws.data_ptr()) % 256 if nb else None
        B.dsa_topk(self.batch, scores, ld or scores.shape[1], k, idx, base, nb)
        return idx

    def mla(self, idx, k=None):
        wl = self.wl
        k = k or idx.shape[1]
        dt = torch.bfloat16 if wl.fp8 else torch.float32
        out = torch.full((self.T, wl.heads, wl.d_v), float("nan"), dtype=dt, device=self.dev)
        lse = torch.full((self.T, wl.heads), float("nan"), device=self.dev)
        ws_bytes = B.dsa_sparse_mla_workspace_size(self.batch, self.mla_dtype, wl.heads, wl.d_qk, wl.d_v, k)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=self.dev)
        B.dsa_sparse_mla_fwd(self.batch, self.layout, self.mla_dtype, wl.heads, wl.d_qk, wl.d_v, self.q, self.kv,
                             idx, k, wl.sm_scale, out, lse, ws, ws_bytes)
        return out, lse

    def forward(self, keep=True):
        wl = self.wl
        dt = torch.bfloat16 if wl.fp8 else torch.float32
        scores = torch.full((self.T, self.ld), float("nan"), device=self.dev) if keep else None
        idx = torch.full((self.T, wl.top_k), -7, dtype=torch.int32, device=self.dev) if keep else None
        out = torch.full((self.T, wl.heads, wl.d_v), float("nan"), dtype=dt, device=self.dev)
        lse = torch.full((self.T, wl.heads), float("nan"), device=self.dev)
        args = B.forward_args(self.batch, self.layout, index_dtype=self.index_dtype, h_i=wl.h_i, d_i=wl.d_i,
                              q_idx=self.qi, q_scale=self.qs, w=self.w, k_idx=self.ki, k_scale=self.ks,
                              index_scale=wl.index_scale, top_k=wl.top_k, scores=scores, ld_scores=self.ld,
                              indices=idx, mla_dtype=self.mla_dtype, heads=wl.heads, d_qk=wl.d_qk, d_v=wl.d_v,
                              q=self.q, kv=self.kv, sm_scale=wl.sm_scale, out=out, lse=lse)
        nbytes = B.dsa_forward_workspace_size(args)
        ws = torch.empty(max(nbytes, 256) + 256, dtype=torch.uint8, device=self.dev)
        base = ws.data_ptr()
        aligned = (base + 255) // 256 * 256
        B.dsa_forward(args, aligned, nbytes)
        return scores, idx, out, lse

    # ---------------- oracle side ----------------
    def seq_keys(self, b):
        lo = int(self.lay.k_seq_start[b])
        return self.ki_hat[lo:lo + int(self.lay.k_len[b])]

    def seq_kv(self, b):
        lo = int(self.lay.k_seq_start[b])
        return self.kv_hat[lo:lo + int(self.lay.k_len[b])]

    def ref_scores(self, t):
        b, p, n = self.rows[t]
        return O.indexer_scores(self.qi_hat[t], self.w_host[t], self.seq_keys(b)[:n], self.wl.index_scale)


def check_indexer(case, scores_gpu, rows):
    """Indexer parity on the given rows; returns the oracle scores by row."""
    got_all = scores_gpu.cpu().numpy()
    refs = {}
    worst = 0.0
    for t in rows:
        b, p, n = case.rows[t]
        ref = case.ref_scores(t)
        got = got_all[t, :n].astype(np.float64)
        assert not np.isnan(got).any(), "row %d: unwritten or NaN scores" % t
        worst = max(worst, indexer_margin(got, ref, t))
        refs[t] = ref
    report("indexer", case.wl.name, worst)
    return refs


def indexer_margin(got, ref, t):
    """Worst |I_gpu - I_ref| / tolerance of one row (asserts it is <= 1)."""
    tol = IDX_RTOL * np.abs(ref) + IDX_FLOOR * np.abs(ref).max()
    d = np.abs(got - ref)
    bad = d > tol
    assert not bad.any(), "row %d: %d scores off, worst |d|=%g at s=%d (ref %g)" % (
        t, bad.sum(), d.max(), int(np.argmax(d)), ref[np.argmax(d)])
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(tol > 0, d / tol, 0.0)
    return float(r.max()) if r.size else 0.0


def report(what, case, ratio):
    """Prints the worst error / tolerance ratio of a parity check (pytest -s shows it)."""
    print("[margin] %s %s: worst error / tolerance = %.3g" % (what, case, ratio), flush=True)


def check_topk_exact(case, scores_gpu, idx_gpu, rows, k=None):
    """GPU top-k equals the oracle's top-k of the same (GPU) score array."""
    k = k or case.wl.top_k
    s_all = scores_gpu.cpu().numpy()
    i_all = idx_gpu.cpu().numpy()
    for t in rows:
        n = case.rows[t][2]
        want = O.topk_indices(s_all[t, :n].astype(np.float64), k)
        assert np.array_equal(i_all[t].astype(np.int64), want), "row %d: top-k differs" % t


def check_topk_end_to_end(case, ref_scores, idx_gpu, rows):
    """Index sets may differ from the oracle's only at near-ties of the k-th score."""
    k = case.wl.top_k
    i_all = idx_gpu.cpu().numpy()
    for t in rows:
        n = case.rows[t][2]
        ref = ref_scores[t]
        m = min(k, n)
        got = i_all[t]
        assert (got[m:] == -1).all() and (np.diff(got[:m]) > 0).all() and got[:m].min() >= 0 and got[m - 1] < n
        want = O.topk_indices(ref, k)
        diff = np.setxor1d(got[:m], want[:m])
        if diff.size:
            tau = ref[want[:m]].min()
            assert (np.abs(ref[diff] - tau) <= TIE_RTOL * abs(tau)).all(), "row %d: selection differs beyond ties" % t


def check_mla(case, idx_gpu, out_gpu, lse_gpu, rows, tol=None):
    """Attention parity, with the oracle run on the GPU's own indices."""
    tol = tol or (ATTN_TOL_BF16 if case.wl.fp8 else ATTN_TOL_F32)
    i_all = idx_gpu.cpu().numpy()
    o_all = out_gpu.float().cpu().numpy()
    l_all = lse_gpu.cpu().numpy()
    worst = worst_lse = 0.0
    for t in rows:
        b, p, n = case.rows[t]
        o_ref, lse_ref = O.sparse_mla(case.q_hat[t], case.seq_kv(b)[:n], i_all[t], case.wl.d_v, case.wl.sm_scale)
        o = o_all[t].astype(np.float64)
        assert not np.isnan(o).any(), "row %d: NaN in output" % t
        err = np.abs(o - o_ref).max() / max(np.abs(o_ref).max(), 1e-30)
        worst = max(worst, err)
        assert err <= tol, "row %d: attention error %g > %g" % (t, err, tol)
        dl = np.abs(l_all[t] - lse_ref).max()
        worst_lse = max(worst_lse, dl)
        assert dl <= LSE_TOL, "row %d: lse off by %g" % (t, dl)
    report("attention", case.wl.name, worst / tol)
    report("lse", case.wl.name, worst_lse / LSE_TOL)
    return worst
