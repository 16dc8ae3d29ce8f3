"""A decode batch (one query row per sequence) declared with
max_q_per_seq = 1 lets the kernels map row t to sequence t directly; the
same batch declared with a looser bound (2, still valid: the bound only has
to cover every sequence's count) takes the general sequence search.  Both
must give the same indices, outputs and lse bit for bit, with contiguous
keys and with 64-token pages (histories past 32768, so that top-k also runs
its two-pass form)."""

import pytest
import torch

from sparse_attention_long_fp8_amd import binding as B
from sparse_attention_long_fp8_amd import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _forward(case, batch):
    wl = case.wl
    out = torch.full((case.T, wl.heads, wl.d_v), float("nan"), dtype=torch.bfloat16, device=case.dev)
    lse = torch.full((case.T, wl.heads), float("nan"), device=case.dev)
    idx = torch.full((case.T, wl.top_k), -7, dtype=torch.int32, device=case.dev)
    args = B.forward_args(batch, case.layout, index_dtype=case.index_dtype, h_i=wl.h_i, d_i=wl.d_i,
                          q_idx=case.qi, q_scale=case.qs, w=case.w, k_idx=case.ki, k_scale=case.ks,
                          index_scale=wl.index_scale, top_k=wl.top_k, scores=None, ld_scores=case.ld,
                          indices=idx, mla_dtype=case.mla_dtype, heads=wl.heads, d_qk=wl.d_qk, d_v=wl.d_v,
                          q=case.q, kv=case.kv, sm_scale=wl.sm_scale, out=out, lse=lse)
    nb = B.dsa_forward_workspace_size(args)
    ws = torch.empty(nb + 256, dtype=torch.uint8, device=case.dev)
    B.dsa_forward(args, ws.data_ptr() + (-ws.data_ptr()) % 256, nb)
    torch.cuda.synchronize()
    return idx, out, lse


@pytest.mark.parametrize("paged", [False, True])
def test_decode_batch_bound_does_not_change_results(paged, gpu):
    if paged:
        wl = synth.Workload("decode_bound_paged", 41, "decode", 6, 0, ctx_range=(3000, 40000), paged=True, top_k=2048)
    else:
        wl = synth.Workload("decode_bound_contig", 42, "decode", 10, 9000, top_k=1024)
    print("\n[decode-bound] %s, %d queries" % (wl.name, wl.batch), flush=True)
    case = H.GpuCase(wl, gpu)
    bt = case.batch
    assert bt.max_q_per_seq == 1 and bt.num_queries == bt.num_seqs
    loose = B.dsa_batch_t(bt.num_seqs, bt.num_queries, bt.q_seq_start, bt.k_len, 2, bt.max_k_len)
    ia, oa, la = _forward(case, bt)
    ib, ob, lb = _forward(case, loose)
    assert torch.equal(ia, ib), "indices differ"
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)), "outputs differ"
    assert torch.equal(la, lb), "lse differs"
    assert bool((ia >= 0).all()), "every row has more candidates than k"
    assert torch.isfinite(oa.float()).all()
