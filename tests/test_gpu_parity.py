"""Parity of the HIP path with the CPU oracle on seeded inputs, stage by stage
and end to end, through the C ABI.  Sizes here let the oracle check every
row while spanning several tiles and a ragged tail; full workload sizes are
in test_gpu_full.py."""

import numpy as np
import pytest
import torch

from sparse_attention_long_fp8_amd import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

W = synth.Workload
SMALL = {
    # the tiny fp32 workload, exactly as measured (L=512, H_I=4 x 32, k=64, 4 heads 80/64)
    "tiny_prefill": synth.WORKLOADS["tiny_prefill"],
    # FP8 / bf16 shapes of the large workloads at a size the oracle checks in full:
    # 300 rows -> several 32-key tiles and a ragged tail; k=64 < n for most rows
    "prefill_300": W("prefill_300", 10, "prefill", 1, 300, top_k=64),
    # ragged decode, contiguous cache, k=256
    "decode_ragged": W("decode_ragged", 11, "decode", 5, 0, ctx_range=(100, 3000), top_k=256),
    # ragged decode from a permuted 64-token page pool with poisoned tails
    "decode_paged": W("decode_paged", 12, "decode", 4, 0, ctx_range=(70, 2000), paged=True, top_k=128),
    # chunked prefill: 40 new queries after a cached prefix, two sequences
    "chunk_2x40": W("chunk_2x40", 13, "chunk", 2, 0, ctx_range=(200, 700), q_per_seq=40, top_k=96),
    # single-head page form: H_I = 32 (smallest FP8 head count), 1/sqrt(d_I) scale, 16 MLA heads
    "prefill_h32": W("prefill_h32", 14, "prefill", 1, 200, h_i=32, top_k=50, heads=16,
                     index_scale=1.0 / np.sqrt(128)),
    # the other MLA head counts: 64 (one workgroup per row and range) and 32
    "decode_h64": W("decode_h64", 17, "decode", 3, 0, ctx_range=(300, 1500), top_k=192, heads=64),
    "prefill_h32mla": W("prefill_h32mla", 18, "prefill", 1, 160, top_k=100, heads=32),
    # the other FP8 indexer head counts on the staged kernel: 128 heads (decode, and a chunk of 24 queries per
    # sequence, which the tiled kernel does not take at 128 heads) and 32 heads over paged keys
    "decode_hi128": W("decode_hi128", 24, "decode", 3, 0, ctx_range=(300, 2500), h_i=128, top_k=128),
    "chunk_hi128": W("chunk_hi128", 25, "chunk", 2, 0, ctx_range=(300, 900), q_per_seq=24, h_i=128, top_k=64,
                     heads=16),
    "decode_hi32_paged": W("decode_hi32_paged", 26, "decode", 3, 0, ctx_range=(70, 1500), paged=True, h_i=32,
                           top_k=64),
    # chunked prefill over paged keys (the tiled indexer kernel resolving page bases; poisoned page tails)
    "chunk_paged": W("chunk_paged", 27, "chunk", 2, 0, ctx_range=(300, 900), q_per_seq=40, paged=True, top_k=96),
    # fp32 path away from the tiny shape: odd sizes (7 x 100 indexer, 5 heads, 53-wide keys, 40-wide values:
    # scalar gathers) in chunks, and the largest fp32 shape (64 x 128 indexer, 64 heads, 256 / 192) over pages
    "f32_chunk_odd": W("f32_chunk_odd", 28, "chunk", 3, 0, ctx_range=(60, 500), q_per_seq=6, h_i=7, d_i=100,
                       fp8=False, top_k=48, heads=5, d_c=40, d_r=13),
    "f32_paged_max": W("f32_paged_max", 29, "decode", 4, 0, ctx_range=(70, 900), paged=True, h_i=64, d_i=128,
                       fp8=False, top_k=100, heads=64, d_c=192, d_r=64),
    # selections longer than the 2048 slots one attention workgroup resolves: two ranges and a merge even in
    # prefill (and the fused indexer -> top-k at k = 2200), and 32 ranges a row for two decodes at k = 4096
    "prefill_k2200": W("prefill_k2200", 30, "prefill", 1, 2600, top_k=2200, heads=16),
    "decode_k4096": W("decode_k4096", 33, "decode", 2, 0, ctx_range=(5000, 9000), top_k=4096),
}


@pytest.fixture(scope="module", params=sorted(SMALL))
def case(request, gpu):
    print("\n[case] %s" % request.param, flush=True)
    return H.GpuCase(SMALL[request.param], gpu)


def test_stages(case):
    rows = list(range(case.T))
    scores = case.indexer()
    refs = H.check_indexer(case, scores, rows)
    idx = case.topk(scores)
    H.check_topk_exact(case, scores, idx, rows)
    H.check_topk_end_to_end(case, refs, idx, rows)
    out, lse = case.mla(idx)
    worst = H.check_mla(case, idx, out, lse, rows)
    print("[%s] worst attention error %.3g" % (case.wl.name, worst))


def test_forward_equals_stages_and_is_deterministic(case):
    s1, i1, o1, l1 = case.forward()
    s2, i2, o2, l2 = case.forward()
    assert torch.equal(i1, i2) and torch.equal(o1.view(torch.int16) if o1.dtype == torch.bfloat16 else o1,
                                               o2.view(torch.int16) if o2.dtype == torch.bfloat16 else o2)
    scores = case.indexer()
    n_of = [r[2] for r in case.rows]
    for t in range(case.T):
        assert torch.equal(scores[t, :n_of[t]], s1[t, :n_of[t]])
    idx = case.topk(scores)
    assert torch.equal(idx, i1)
    out, lse = case.mla(idx)
    assert torch.equal(out.float(), o1.float()) and torch.equal(lse, l1)
    # the internal-workspace variant gives the same result
    _, _, o3, l3 = case.forward(keep=False)
    assert torch.equal(o3.float(), o1.float()) and torch.equal(l3, l1)


def test_paged_equals_contiguous(gpu):
    wl = SMALL["decode_paged"]
    paged = H.GpuCase(wl, gpu)
    flat = H.GpuCase(wl, gpu, force_contiguous=True)
    sp, ip, op, lp = paged.forward()
    sf, if_, of, lf = flat.forward()
    for t in range(paged.T):
        n = paged.rows[t][2]
        assert torch.equal(sp[t, :n], sf[t, :n])
    assert torch.equal(ip, if_)
    assert torch.equal(op.float(), of.float()) and torch.equal(lp, lf)


def test_k_at_least_context_is_dense_attention(gpu):
    """With k >= every n_t the selection is all of 0..t and attention is dense causal."""
    from oracle import dsa_oracle as O
    wl = W("dense_check", 15, "prefill", 1, 96, top_k=128)
    c = H.GpuCase(wl, gpu)
    _, idx, out, lse = c.forward()
    i = idx.cpu().numpy()
    for t in range(c.T):
        assert i[t, :t + 1].tolist() == list(range(t + 1)) and (i[t, t + 1:] == -1).all()
    o_d, lse_d = O.dense_causal_mla(c.q_hat[:24], c.kv_hat[:24], wl.d_v, wl.sm_scale)
    o = out.float().cpu().numpy()[:24]
    assert np.abs(o - o_d).max() / np.abs(o_d).max() <= H.ATTN_TOL_BF16
    assert np.abs(lse.cpu().numpy()[:24] - lse_d).max() <= H.LSE_TOL


def test_wide_logit_range(gpu):
    """Queries scaled by 32 (exact in bf16): the logits of a row spread over
    hundreds of log2 units, so later tiles exceed a head's running reference
    max by far more than the kernel's headroom and its rescale path runs,
    several times per range.  Rows here have one slot range of 32 tiles."""
    wl = W("chunk_wide", 16, "chunk", 2, 0, ctx_range=(1500, 2500), q_per_seq=64, top_k=1024)
    c = H.GpuCase(wl, gpu)
    idx = c.topk(c.indexer())
    c.q = (c.q.float() * 32).to(torch.bfloat16)
    c.q_hat = c.q_hat * 32
    out, lse = c.mla(idx)
    rows = list(range(0, c.T, 3))
    worst = H.check_mla(c, idx, out, lse, rows)
    print("[chunk_wide] worst attention error %.3g" % worst)
