"""Fused indexer -> top-k (dsa_indexer_topk): the positions it writes must be
exactly those of the two separate stages (dsa_indexer_scores, then
dsa_topk) on the same inputs -- the fused kernel computes the same scores
and selects from bounded candidate lists -- and, end to end, agree with the
oracle's selection on the oracle's scores up to near-ties of the k-th score.
Cases: a causal prefill with several compactions of every long row's list
(k = 512 and k = 64), ragged chunked prefill over three sequences, the same
two shapes over a paged cache (pages scattered over the pool), 128 and 32
indexer heads (one and two rows a wave), and rows made all ties (zero head
weights), where the k lowest positions must win."""

import numpy as np
import pytest
import torch

from sparse_attention_long_fp8_amd import binding as B
from sparse_attention_long_fp8_amd import synth

from .helpers import GpuCase, check_topk_end_to_end

pytestmark = pytest.mark.gpu

CASES = {
    "prefill_3000_k512": synth.Workload("fused_prefill", 31, "prefill", 1, 3000, top_k=512, heads=16),
    "prefill_1500_k64": synth.Workload("fused_prefill_k64", 33, "prefill", 1, 1500, top_k=64, heads=16),
    "chunk_3seq_k256": synth.Workload("fused_chunk", 32, "chunk", 3, 0, ctx_range=(900, 2500), q_per_seq=40,
                                      top_k=256, heads=16),
    "prefill_paged_2500_k128": synth.Workload("fused_prefill_paged", 34, "prefill", 1, 2500, top_k=128, heads=16,
                                              paged=True),
    "chunk_paged_3seq_k256": synth.Workload("fused_chunk_paged", 35, "chunk", 3, 0, ctx_range=(900, 2500),
                                            q_per_seq=40, top_k=256, heads=16, paged=True),
    "prefill_h128_2000_k128": synth.Workload("fused_prefill_h128", 36, "prefill", 1, 2000, h_i=128, top_k=128,
                                             heads=16),
    "chunk_h32_paged_k64": synth.Workload("fused_chunk_h32", 37, "chunk", 3, 0, ctx_range=(700, 1800),
                                          q_per_seq=24, h_i=32, top_k=64, heads=16, paged=True),
}


def _fused(case, k, w=None):
    wl = case.wl
    ws_bytes = B.dsa_indexer_topk_workspace_size(case.batch, case.layout, case.index_dtype, wl.h_i, wl.d_i, k)
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=case.dev)
    base = ws.data_ptr()
    aligned = base + (-base) % 256
    idx = torch.full((case.T, k), -7, dtype=torch.int32, device=case.dev)
    B.dsa_indexer_topk(case.batch, case.layout, case.index_dtype, wl.h_i, wl.d_i, case.qi, case.qs,
                       case.w if w is None else w, case.ki, case.ks, wl.index_scale, k, idx, aligned, ws_bytes)
    torch.cuda.synchronize()
    return idx


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request, gpu):
    return GpuCase(CASES[request.param], gpu)


def test_fused_equals_separate_stages(case):
    k = case.wl.top_k
    assert case.lay.max_q_per_seq >= 8 and case.lay.max_k_len <= 131072  # the fused kernel applies
    got = _fused(case, k).cpu().numpy()
    want = case.topk(case.indexer(), k=k).cpu().numpy()
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, "rows %s differ (first: got %s want %s)" % (bad[:5], got[bad[0]][:8], want[bad[0]][:8])


def test_fused_matches_oracle_end_to_end(case):
    idx = _fused(case, case.wl.top_k)
    T = case.T
    rows = sorted({0, 1, T // 3, T // 2, T - 2, T - 1})
    refs = {t: case.ref_scores(t) for t in rows}
    check_topk_end_to_end(case, refs, idx, rows)


def test_fused_all_ties_keep_lowest_positions(case):
    k = case.wl.top_k
    zero_w = torch.zeros_like(case.w)  # every score is exactly 0
    got = _fused(case, k, w=zero_w).cpu().numpy()
    for t, (b, p, n) in enumerate(case.rows):
        m = min(k, n)
        assert (got[t, :m] == np.arange(m)).all(), "row %d" % t
        assert (got[t, m:] == -1).all(), "row %d padding" % t
