"""Parity at the measured workloads' full sizes, in the launch configuration
bench.py times.  The oracle checks sampled rows one by one (every row of the
32-query decode); properties that hold at any size (exactly min(k, n_t)
indices, ascending, causal, -1 padding, finite outputs, no read of poisoned
cache slots) are checked on every row."""

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from sparse_attention_long_fp8_amd import synth
from bench import prefill_sample_rows
from sparse_attention_long_fp8_amd.workload import DeviceWorkload
from tests import helpers as H

pytestmark = pytest.mark.gpu

FULL = ["decode_32k", "prefill_16k", "prefill_64k", "paged_decode"]


def _sample(wl, rows):
    """Every row of the decode workloads; on the prefills the rows at the ends
    and around the k boundary plus seeded rows in equal strata (the 64k
    prefill: 256 rows drawn like the benchmark's oracle sample, with another
    seed)."""
    T = len(rows)
    if wl.kind == "decode":
        return list(range(T))
    fixed, strat = prefill_sample_rows(T, wl.top_k, 256 if T > 16384 else 64, seed=123)
    return sorted(set(fixed) | set(strat))


class RowOracle:
    """Oracle inputs of single rows, regenerated from the seeded generator."""

    def __init__(self, dw):
        self.dw = dw
        self.s = dw.synth
        self.rows = O.query_rows(dw.lay.q_seq_start, dw.lay.k_len)
        self._seq = {}

    def seq(self, b):
        if b not in self._seq:
            if len(self._seq) > 2:
                self._seq.clear()
            lay, wl = self.dw.lay, self.dw.wl
            base, n = int(lay.k_seq_start[b]), int(lay.k_len[b])
            kc, ks = self.s.ki(base, base + n)
            self._seq[b] = (O.dequant_e4m3(kc, ks), O.decode_bf16(self.s.kv(base, base + n)))
        return self._seq[b]

    def prefetch(self, rows):
        """Regenerates the query-side inputs of `rows` in parallel (each row
        redraws its 256-row chunk, so one at a time is slow)."""
        from concurrent.futures import ThreadPoolExecutor

        def one(t):
            qc, qs = self.s.qi(t, t + 1)
            return (O.dequant_e4m3(qc, qs)[0], self.s.w(t, t + 1)[0].astype(np.float64),
                    O.decode_bf16(self.s.q(t, t + 1))[0])

        with ThreadPoolExecutor(16) as ex:
            self._q = dict(zip(rows, ex.map(one, rows)))

    def row(self, t):
        b, p, n = self.rows[t]
        if t in getattr(self, "_q", {}):
            qi_h, w, q_h = self._q.pop(t)
        else:
            qc, qs = self.s.qi(t, t + 1)
            qi_h, w, q_h = (O.dequant_e4m3(qc, qs)[0], self.s.w(t, t + 1)[0].astype(np.float64),
                            O.decode_bf16(self.s.q(t, t + 1))[0])
        keys, kv = self.seq(b)
        return qi_h, w, keys[:n], q_h, kv[:n], n


@pytest.fixture(scope="module", params=FULL)
def full(request, gpu):
    wl = synth.WORKLOADS[request.param]
    print("\n[full] %s" % wl.name, flush=True)
    dw = DeviceWorkload(wl, gpu)
    dw.step()
    torch.cuda.synchronize()
    yield dw
    del dw
    torch.cuda.empty_cache()


def test_every_row_properties(full):
    dw = full
    wl = dw.wl
    rows = O.query_rows(dw.lay.q_seq_start, dw.lay.k_len)
    n = torch.tensor([r[2] for r in rows], dtype=torch.int64, device=dw.dev)
    k = wl.top_k
    idx = dw.idx.long()
    m = torch.clamp(n, max=k)
    slot = torch.arange(k, device=dw.dev)[None, :]
    live = slot < m[:, None]
    assert bool((idx[live] >= 0).all()) and bool((idx[~live] == -1).all()), "wrong count or padding"
    assert bool((idx < n[:, None])[live].all()), "an index beyond the causal bound"
    asc = (idx[:, 1:] > idx[:, :-1]) | ~live[:, 1:]
    assert bool(asc.all()), "indices not strictly ascending"
    assert bool(torch.isfinite(dw.out.float()).all()) and bool(torch.isfinite(dw.lse).all())
    # every written score is finite (poisoned paged slots were never read)
    for r0 in range(0, dw.T, 1024):
        r1 = min(dw.T, r0 + 1024)
        cols = torch.arange(dw.ld, device=dw.dev)[None, :]
        written = cols < n[r0:r1, None]
        blk = dw.scores[r0:r1]
        assert bool(torch.isfinite(blk[written]).all()), "non-finite score in rows %d..%d" % (r0, r1)


def test_sampled_rows_match_oracle(full):
    dw = full
    wl = dw.wl
    ro = RowOracle(dw)
    rows = _sample(wl, ro.rows)
    print("[full] %s: oracle on %d rows" % (wl.name, len(rows)), flush=True)
    ro.prefetch(rows)
    scores = dw.scores
    idx = dw.idx.cpu().numpy()
    worst_att = worst_idx = worst_lse = 0.0
    for t in rows:
        qi_h, w, keys, q_h, kv, n = ro.row(t)
        ref = O.indexer_scores(qi_h, w, keys, wl.index_scale)
        got = scores[t, :n].double().cpu().numpy()
        worst_idx = max(worst_idx, H.indexer_margin(got, ref, t))
        # top-k bit-exact on the GPU's own scores
        assert np.array_equal(idx[t].astype(np.int64), O.topk_indices(got, wl.top_k)), "row %d: top-k" % t
        # end to end: differences only at near-ties of the oracle's k-th score
        m = min(wl.top_k, n)
        want = O.topk_indices(ref, wl.top_k)
        diff = np.setxor1d(idx[t, :m], want[:m])
        if diff.size:
            tau = ref[want[:m]].min()
            assert (np.abs(ref[diff] - tau) <= H.TIE_RTOL * abs(tau)).all(), "row %d: selection beyond ties" % t
        # attention on the GPU's indices
        o_ref, lse_ref = O.sparse_mla(q_h, kv, idx[t], wl.d_v, wl.sm_scale)
        o = dw.out[t].float().cpu().numpy().astype(np.float64)
        err = np.abs(o - o_ref).max() / np.abs(o_ref).max()
        worst_att = max(worst_att, err)
        assert err <= H.ATTN_TOL_BF16, "row %d: attention error %g" % (t, err)
        dl = np.abs(dw.lse[t].cpu().numpy() - lse_ref).max()
        worst_lse = max(worst_lse, dl)
        assert dl <= H.LSE_TOL, "row %d: lse" % t
    print("[full] %s: worst attention error %.3g" % (wl.name, worst_att), flush=True)
    H.report("indexer", wl.name, worst_idx)
    H.report("attention", wl.name, worst_att / H.ATTN_TOL_BF16)
    H.report("lse", wl.name, worst_lse / H.LSE_TOL)


def test_needles_are_selected(full):
    dw = full
    if dw.wl.needles == 0:
        pytest.skip("workload has no planted needles")
    idx = dw.idx.cpu().numpy()
    for b in range(dw.wl.batch):
        t = int(dw.lay.q_seq_start[b + 1]) - 1
        missing = set(dw.lay.needle_pos[b].tolist()) - set(idx[t].tolist())
        assert not missing, "sequence %d: needles %s not selected" % (b, sorted(missing))


def test_fused_forward_equals_stages(full):
    dw = full
    idx0, out0, lse0 = dw.idx.clone(), dw.out.clone(), dw.lse.clone()
    dw.forward()
    torch.cuda.synchronize()
    assert torch.equal(dw.idx, idx0)
    assert torch.equal(dw.out.view(torch.int16), out0.view(torch.int16)) and torch.equal(dw.lse, lse0)


def test_forward_without_kept_scores_equals_stages(full):
    """dsa_forward with no score array (prefill: the fused indexer -> top-k
    kernel) selects exactly the stages' indices and so gives the same output."""
    dw = full
    dw.step()
    idx0, out0, lse0 = dw.idx.clone(), dw.out.clone(), dw.lse.clone()
    dw.idx.fill_(-7)
    dw.forward(keep_scores=False)
    torch.cuda.synchronize()
    assert torch.equal(dw.idx, idx0)
    assert torch.equal(dw.out.view(torch.int16), out0.view(torch.int16)) and torch.equal(dw.lse, lse0)
