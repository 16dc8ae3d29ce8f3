"""A workload resident on the GPU: seeded inputs uploaded into device tensors,
the batch / cache descriptors, output buffers, and the three stage calls
through the C ABI.  The benchmark and the full-size tests share it, so the
tests check exactly the launch configuration that is timed."""

from __future__ import annotations

import numpy as np
import torch

from . import binding as B
from . import synth


def _i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def _bf16(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


class DeviceWorkload:
    """Inputs of one workload on `dev` (optionally several copies, rotated by
    the benchmark so that no step finds its inputs in the last-level cache)."""

    def __init__(self, wl: synth.Workload, dev, copies: int = 1, log=None):
        self.wl = wl
        self.dev = dev
        self.synth = s = synth.Synth(wl)
        lay = self.lay = s.layout
        self.T = T = lay.num_queries
        self.N = N = int(lay.k_seq_start[-1])
        if log:
            log("%s: generating inputs (T=%d, keys=%d)" % (wl.name, T, N))
        self.q_seq_start = _i32(lay.q_seq_start, dev)
        self.k_len = _i32(lay.k_len, dev)
        self.k_seq_start = torch.from_numpy(lay.k_seq_start[:-1].astype(np.int64)).to(dev)
        self.batch = B.make_batch(self.q_seq_start, self.k_len, wl.batch, T, lay.max_q_per_seq, lay.max_k_len)
        self.ld = (lay.max_k_len + 3) // 4 * 4
        self.index_dtype = B.DSA_FP8_E4M3 if wl.fp8 else B.DSA_F32
        self.mla_dtype = B.DSA_BF16 if wl.fp8 else B.DSA_F32
        dt_q = torch.bfloat16 if wl.fp8 else torch.float32
        # query-side inputs, generated in slabs straight into device tensors
        qi = torch.empty((T, wl.h_i, wl.d_i), dtype=torch.uint8 if wl.fp8 else torch.float32, device=dev)
        qs = torch.empty(T, dtype=torch.float32, device=dev) if wl.fp8 else None
        w = torch.empty((T, wl.h_i), dtype=torch.float32, device=dev)
        q = torch.empty((T, wl.heads, wl.d_qk), dtype=dt_q, device=dev)
        slab = 2048
        for r0 in range(0, T, slab):
            r1 = min(T, r0 + slab)
            c, sc = s.qi(r0, r1)
            qi[r0:r1] = torch.from_numpy(c).to(dev)
            if wl.fp8:
                qs[r0:r1] = torch.from_numpy(sc).to(dev)
            w[r0:r1] = torch.from_numpy(s.w(r0, r1)).to(dev)
            qq = s.q(r0, r1)
            q[r0:r1] = _bf16(qq, dev) if wl.fp8 else torch.from_numpy(qq).to(dev)
        # key-side inputs
        if wl.paged:
            ki_pool, ks_pool, kv_pool = s.paged_pools()
            ki = torch.from_numpy(ki_pool).to(dev)
            ks = torch.from_numpy(ks_pool).to(dev)
            kv = _bf16(kv_pool, dev)
            del ki_pool, ks_pool, kv_pool
            self.page_table = _i32(lay.page_table, dev)
            self.layout = B.make_paged_layout(self.page_table, lay.page_table.shape[1], lay.num_pages)
        else:
            ki = torch.empty((N, wl.d_i), dtype=torch.uint8 if wl.fp8 else torch.float32, device=dev)
            ks = torch.empty(N, dtype=torch.float32, device=dev) if wl.fp8 else None
            kv = torch.empty((N, wl.d_qk), dtype=dt_q, device=dev)
            for g0 in range(0, N, 65536):
                g1 = min(N, g0 + 65536)
                c, sc = s.ki(g0, g1)
                ki[g0:g1] = torch.from_numpy(c).to(dev)
                if wl.fp8:
                    ks[g0:g1] = torch.from_numpy(sc).to(dev)
                kk = s.kv(g0, g1)
                kv[g0:g1] = _bf16(kk, dev) if wl.fp8 else torch.from_numpy(kk).to(dev)
            self.layout = B.make_contiguous_layout(self.k_seq_start, N)
        self.sets = [(qi, qs, w, q, ki, ks, kv)]
        for _ in range(copies - 1):
            self.sets.append(tuple(None if x is None else x.clone() for x in self.sets[0]))
        self.copies = copies
        # outputs and workspace
        self.scores = torch.empty((T, self.ld), dtype=torch.float32, device=dev)
        self.idx = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev)
        self.out = torch.empty((T, wl.heads, wl.d_v), dtype=dt_q, device=dev)
        self.lse = torch.empty((T, wl.heads), dtype=torch.float32, device=dev)
        self.ws_bytes = B.dsa_sparse_mla_workspace_size(self.batch, self.mla_dtype, wl.heads, wl.d_qk, wl.d_v,
                                                        wl.top_k)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        # top-k of few long rows runs in two passes over a candidate-list workspace (256-byte aligned)
        self.topk_ws_bytes = B.dsa_topk_workspace_size(self.batch, wl.top_k)
        self.topk_ws = torch.empty(self.topk_ws_bytes + 256, dtype=torch.uint8, device=dev)
        self.topk_ws_ptr = self.topk_ws.data_ptr() + (-self.topk_ws.data_ptr()) % 256

    # ---- the three stages (exactly what dsa_forward enqueues) ----
    def indexer(self, copy=0, stream=None):
        wl = self.wl
        qi, qs, w, _, ki, ks, _ = self.sets[copy % self.copies]
        B.dsa_indexer_scores(self.batch, self.layout, self.index_dtype, wl.h_i, wl.d_i, qi, qs, w, ki, ks,
                             wl.index_scale, self.scores, self.ld, stream=stream)

    def topk(self, stream=None):
        B.dsa_topk(self.batch, self.scores, self.ld, self.wl.top_k, self.idx, self.topk_ws_ptr, self.topk_ws_bytes,
                   stream=stream)

    def mla(self, copy=0, stream=None):
        wl = self.wl
        _, _, _, q, _, _, kv = self.sets[copy % self.copies]
        B.dsa_sparse_mla_fwd(self.batch, self.layout, self.mla_dtype, wl.heads, wl.d_qk, wl.d_v, q, kv, self.idx,
                             wl.top_k, wl.sm_scale, self.out, self.lse, self.ws, self.ws_bytes, stream=stream)

    def step(self, copy=0, stream=None, events=None):
        """One pass of the whole path; events[0..3] are recorded around the stages."""
        if events:
            events[0].record(stream)
        self.indexer(copy, stream)
        if events:
            events[1].record(stream)
        self.topk(stream)
        if events:
            events[2].record(stream)
        self.mla(copy, stream)
        if events:
            events[3].record(stream)

    def prepare_forward(self):
        """Argument blocks of the fused entry point for every input copy, and
        its workspace, built once so that a timed loop only makes the call.
        The scores are not kept, so shapes with a fused indexer -> top-k
        kernel take it (the indices are kept)."""
        wl = self.wl
        self._fwd_args = []
        for qi, qs, w, q, ki, ks, kv in self.sets:
            self._fwd_args.append(B.forward_args(
                self.batch, self.layout, index_dtype=self.index_dtype, h_i=wl.h_i, d_i=wl.d_i, q_idx=qi, q_scale=qs,
                w=w, k_idx=ki, k_scale=ks, index_scale=wl.index_scale, top_k=wl.top_k, scores=None,
                ld_scores=self.ld, indices=self.idx, mla_dtype=self.mla_dtype, heads=wl.heads, d_qk=wl.d_qk,
                d_v=wl.d_v, q=q, kv=kv, sm_scale=wl.sm_scale, out=self.out, lse=self.lse))
        need = max(B.dsa_forward_workspace_size(a) for a in self._fwd_args)
        self._fwd_ws = torch.empty(max(need, 1), dtype=torch.uint8, device=self.dev)
        self._fwd_need = need

    def forward_prepared(self, copy=0, stream=None):
        """One pass through dsa_forward with the prepared arguments."""
        B.dsa_forward(self._fwd_args[copy % self.copies], self._fwd_ws, self._fwd_need, stream=stream)

    def forward(self, copy=0, stream=None, keep_scores=True):
        """The same pass through the fused dsa_forward entry point (without
        kept scores, shapes with a fused indexer -> top-k kernel take it)."""
        wl = self.wl
        qi, qs, w, q, ki, ks, kv = self.sets[copy % self.copies]
        args = B.forward_args(self.batch, self.layout, index_dtype=self.index_dtype, h_i=wl.h_i, d_i=wl.d_i,
                              q_idx=qi, q_scale=qs, w=w, k_idx=ki, k_scale=ks, index_scale=wl.index_scale,
                              top_k=wl.top_k, scores=self.scores if keep_scores else None, ld_scores=self.ld,
                              indices=self.idx,
                              mla_dtype=self.mla_dtype, heads=wl.heads, d_qk=wl.d_qk, d_v=wl.d_v, q=q, kv=kv,
                              sm_scale=wl.sm_scale, out=self.out, lse=self.lse)
        need = B.dsa_forward_workspace_size(args)
        if need > self.ws.numel():
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.dev)
        B.dsa_forward(args, self.ws, need, stream=stream)
