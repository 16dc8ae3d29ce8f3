"""dsa_forward_noalloc (the whole path with its workspace in the library's
static device array) against dsa_forward with a caller workspace: two calls
in a row, the second on a smaller batch, each bit for bit equal to
dsa_forward on the same inputs; and a call whose workspace would exceed the
array is refused before anything is launched."""

import pytest
import torch

from sparse_attention_long_fp8_amd import binding as B
from sparse_attention_long_fp8_amd import synth
from tests import helpers as H

def _run(case, noalloc, keep_indices):
    wl = case.wl
    out = torch.full((case.T, wl.heads, wl.d_v), float("nan"), dtype=torch.bfloat16, device=case.dev)
    lse = torch.full((case.T, wl.heads), float("nan"), device=case.dev)
    idx = torch.full((case.T, wl.top_k), -7, dtype=torch.int32, device=case.dev) if keep_indices else None
    args = B.forward_args(case.batch, case.layout, index_dtype=case.index_dtype, h_i=wl.h_i, d_i=wl.d_i,
                          q_idx=case.qi, q_scale=case.qs, w=case.w, k_idx=case.ki, k_scale=case.ks,
                          index_scale=wl.index_scale, top_k=wl.top_k, scores=None, ld_scores=case.ld,
                          indices=idx, mla_dtype=case.mla_dtype, heads=wl.heads, d_qk=wl.d_qk, d_v=wl.d_v,
                          q=case.q, kv=case.kv, sm_scale=wl.sm_scale, out=out, lse=lse)
    if noalloc:
        B.dsa_forward_noalloc(args)
    else:
        nb = B.dsa_forward_workspace_size(args)
        ws = torch.empty(nb + 256, dtype=torch.uint8, device=case.dev)
        B.dsa_forward(args, ws.data_ptr() + (-ws.data_ptr()) % 256, nb)
        torch.cuda.synchronize()
        del ws
    torch.cuda.synchronize()
    return idx, out, lse


def _same(a, b):
    ia, oa, la = a
    ib, ob, lb = b
    if ia is not None:
        assert torch.equal(ia, ib), "indices differ"
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)), "outputs differ"
    assert torch.equal(la, lb), "lse differs"


@pytest.mark.gpu
def test_noalloc_matches_forward_twice_second_smaller(gpu):
    # first: 12 decodes over 8192 cached tokens (contiguous; the attention
    # splits each selection into ranges, so the array holds scores, indices
    # and split partials); second, smaller: 3 decodes over 64-token pages of
    # 1000-3000 tokens, k = 512, the same array reused
    big = synth.Workload("noalloc_decode", 31, "decode", 12, 8192)
    small = synth.Workload("noalloc_paged", 32, "decode", 3, 0, ctx_range=(1000, 3000), paged=True, top_k=512)
    cases = [H.GpuCase(big, gpu), H.GpuCase(small, gpu)]
    for case, keep in zip(cases, (False, True)):
        print("[noalloc] %s, %d queries, kept indices %s" % (case.wl.name, case.T, keep), flush=True)
        ref = _run(case, noalloc=False, keep_indices=keep)
        got = _run(case, noalloc=True, keep_indices=keep)
        _same(ref, got)
        assert torch.isfinite(got[1].float()).all()
    # the first case again after the smaller one: the array keeps the last
    # call's contents, and nothing of them leaks into a new call
    ref = _run(cases[0], noalloc=False, keep_indices=True)
    _same(ref, _run(cases[0], noalloc=True, keep_indices=True))


def test_noalloc_refuses_a_workspace_beyond_the_array():
    # a 16384-token prefill with its scores (1 GiB) and indices (128 MiB) in
    # the workspace: refused on the host, before any device call
    wl = synth.WORKLOADS["prefill_16k"]
    lay = synth.make_layout(wl)
    bt = B.dsa_batch_t(1, lay.num_queries, 0x1000, 0x2000, lay.max_q_per_seq, lay.max_k_len)
    ly = B.dsa_kv_layout_t(0, 0x3000, None, 0, 64, lay.max_k_len)
    args = B.forward_args(bt, ly, index_dtype=B.DSA_FP8_E4M3, h_i=64, d_i=128, q_idx=0x10, q_scale=0x20, w=0x30,
                          k_idx=0x40, k_scale=0x50, index_scale=1.0, top_k=2048, scores=None, ld_scores=16384,
                          indices=None, mla_dtype=B.DSA_BF16, heads=128, d_qk=576, d_v=512, q=0x60, kv=0x70,
                          sm_scale=0.04, out=0x80)
    assert B.dsa_forward_workspace_size(args) > 96 << 20
    # nothing is launched (the pointers are fake, never dereferenced)
    st = B.dsa_forward_noalloc(args, check=False)
    assert st == B.DSA_ERR_WORKSPACE_TOO_SMALL
    assert "static scratch" in B.dsa_last_error()
