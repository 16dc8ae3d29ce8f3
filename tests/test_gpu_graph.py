"""dsa_forward under HIP graph capture: the path allocates, frees and
synchronises nothing and clears no memory with memset, so one call can be
captured and replayed.  Each replay must reproduce the eager result bit for
bit (the kernels are deterministic), with eager passes on other inputs and
host synchronisations between the replays, and the outputs clobbered before
each replay so that a replay that writes nothing cannot pass."""

import pytest
import torch

from sparse_attention_long_fp8_amd import synth
from sparse_attention_long_fp8_amd.workload import DeviceWorkload

pytestmark = pytest.mark.gpu

W = synth.Workload
CASES = {
    "decode_ragged": W("graph_decode", 21, "decode", 6, 0, ctx_range=(100, 3000), top_k=256),
    "prefill_fused": W("graph_prefill", 22, "prefill", 1, 700, top_k=128, heads=16),
    "decode_paged": W("graph_paged", 23, "decode", 4, 0, ctx_range=(70, 2000), paged=True, top_k=128),
}


def _outputs(dw):
    return dw.idx.clone(), dw.out.clone(), dw.lse.clone()


def _same(dw, ref):
    idx, out, lse = ref
    return (torch.equal(dw.idx, idx) and torch.equal(dw.out.view(torch.int16), out.view(torch.int16))
            and torch.equal(dw.lse, lse))


@pytest.mark.parametrize("name", sorted(CASES))
def test_captured_forward_replays_match_eager(gpu, name):
    print("\n[graph] %s" % name, flush=True)
    dw = DeviceWorkload(CASES[name], gpu, copies=2)
    # the second copy gets other head weights, so its selection differs
    gen = torch.Generator(device=gpu).manual_seed(7)
    w1 = dw.sets[1][2]
    w1.copy_(torch.rand(w1.shape, device=gpu, generator=gen))
    dw.prepare_forward()
    ref = []
    for c in range(2):
        dw.forward_prepared(c)
        torch.cuda.synchronize()
        ref.append(_outputs(dw))
    assert not torch.equal(ref[0][0], ref[1][0]), "the two input copies must select differently"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dw.forward_prepared(0)
    torch.cuda.synchronize()
    for r in range(3):
        dw.idx.fill_(-7)
        dw.out.fill_(float("nan"))
        dw.lse.fill_(float("nan"))
        dw.forward_prepared(1)          # eager work on other inputs between replays
        torch.cuda.synchronize()
        assert _same(dw, ref[1]), "eager pass %d" % r
        dw.idx.fill_(-7)
        dw.out.fill_(float("nan"))
        dw.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(dw, ref[0]), "replay %d differs from the eager result" % r
