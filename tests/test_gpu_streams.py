"""Calls on different streams may run concurrently: the library keeps no
global mutable state, and each call has its own workspace.  Two dsa_forward
calls on two streams (default priority), issued back to back without waiting,
must give bit for bit what each gives alone.  Outputs are allocated on the
stream that uses them, and the inputs are complete before either stream
starts."""

import pytest
import torch

from sparse_attention_long_fp8_amd import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

W = synth.Workload
A = W("streams_decode", 31, "decode", 5, 0, ctx_range=(300, 3000), top_k=256)
Bw = W("streams_prefill", 32, "prefill", 1, 600, top_k=96)


def _bits(t):
    # bit patterns: the kept scores are NaN past each row's n_t (left unwritten), and NaN != NaN
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _same(x, y):
    return all(u is None and v is None or torch.equal(_bits(u), _bits(v)) for u, v in zip(x, y))


@pytest.mark.parametrize("keep", [True, False])
def test_two_streams_match_sequential(gpu, keep):
    print("\n[streams] keep=%s" % keep, flush=True)
    a = H.GpuCase(A, gpu)
    b = H.GpuCase(Bw, gpu)
    ref_a = a.forward(keep=keep)
    ref_b = b.forward(keep=keep)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for r in range(3):
        with torch.cuda.stream(s1):
            got_a = a.forward(keep=keep)
        with torch.cuda.stream(s2):
            got_b = b.forward(keep=keep)
        torch.cuda.synchronize()
        assert _same(got_a, ref_a), "stream 1, round %d" % r
        assert _same(got_b, ref_b), "stream 2, round %d" % r
