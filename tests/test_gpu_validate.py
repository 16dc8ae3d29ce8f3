"""dsa_validate: the on-request check of device-side preconditions.  Valid
batches (contiguous and paged, with selected positions and scores) report
nothing; each planted violation is reported with its code and location.
Every planted value is only read and compared by the checker, which never
forms an address from it."""

import numpy as np
import pytest
import torch

from sparse_attention_long_fp8_amd import binding as B

pytestmark = pytest.mark.gpu

K_LEN = [100, 300, 50]
NQ = [2, 5, 1]
MAXK = 300
K = 64
PS = 64


def _rows():
    """(sequence, n_t) of every query row."""
    out = []
    for b, (kl, nq) in enumerate(zip(K_LEN, NQ)):
        for i in range(nq):
            out.append((b, kl - nq + i + 1))
    return out


class Case:
    def __init__(self, gpu, paged=False, k_len=None, q_seq_start=None, k_seq_start=None, page_fix=None,
                 index_fix=None, score_fix=None):
        rng = np.random.default_rng(5)
        self.gpu = gpu
        k_len = list(K_LEN if k_len is None else k_len)
        qss = np.concatenate([[0], np.cumsum(NQ)]).astype(np.int32) if q_seq_start is None else \
            np.asarray(q_seq_start, np.int32)
        T = int(sum(NQ))
        t_ = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
        self.qs, self.kl = t_(qss), t_(np.asarray(k_len, np.int32))
        self.batch = B.make_batch(self.qs, self.kl, len(K_LEN), T, max(NQ), MAXK)
        if paged:
            pages = [-(-n // PS) for n in K_LEN]
            self.P = sum(pages)
            stride = max(pages)
            table = -np.ones((len(K_LEN), stride), np.int32)
            ids = rng.permutation(self.P).astype(np.int32)
            c = 0
            for b, n in enumerate(pages):
                table[b, :n] = ids[c:c + n]
                c += n
            if page_fix:
                table[page_fix[0], page_fix[1]] = page_fix[2]
            self.tab = t_(table)
            self.layout = B.make_paged_layout(self.tab, stride, self.P, PS)
        else:
            kss = np.concatenate([[0], np.cumsum(K_LEN)[:-1]]).astype(np.int64) if k_seq_start is None else \
                np.asarray(k_seq_start, np.int64)
            self.ks = t_(kss)
            self.layout = B.make_contiguous_layout(self.ks, int(sum(K_LEN)))
        idx = -np.ones((T, K), np.int32)
        scores = np.full((T, MAXK), np.nan, np.float32)   # NaN past n_t is allowed
        for t, (b, n) in enumerate(_rows()):
            m = min(K, n)
            idx[t, :m] = np.sort(rng.choice(n, m, replace=False))
            scores[t, :n] = rng.standard_normal(n).astype(np.float32)
        if index_fix:
            idx[index_fix[0], index_fix[1]] = index_fix[2]
        if score_fix:
            scores[score_fix[0], score_fix[1]] = np.nan
        self.idx, self.scores = t_(idx), t_(scores)
        self.report = torch.full((4,), 7, dtype=torch.int32, device=gpu)

    def run(self, layout=True, indices=True, scores=True):
        B.dsa_validate(self.batch, self.layout if layout else None, self.idx if indices else None, K,
                       self.scores if scores else None, MAXK, self.report)
        torch.cuda.synchronize()
        return self.report.cpu().numpy().tolist()


def test_valid_batches_report_nothing(gpu):
    assert Case(gpu).run() == [0, 0, 0, 0]
    assert Case(gpu, paged=True).run() == [0, 0, 0, 0]
    assert Case(gpu).run(layout=False, indices=False, scores=False) == [0, 0, 0, 0]


def test_batch_arrays(gpu):
    # history longer than max_k_len
    assert Case(gpu, k_len=[100, MAXK + 1, 50]).run() == [B.DSA_CHECK_BATCH, 1, NQ[1], MAXK + 1]
    # more queries than history
    assert Case(gpu, k_len=[100, 300, 0]).run()[:2] == [B.DSA_CHECK_BATCH, 2]
    # q_seq_start not ending at num_queries
    r = Case(gpu, q_seq_start=[0, 2, 7, 9]).run()
    assert r[:2] == [B.DSA_CHECK_BATCH, 2]


def test_rows_and_pages(gpu):
    # contiguous rows past the end of the cache (k_seq_start[2] + 50 > 450)
    assert Case(gpu, k_seq_start=[0, 100, 401]).run() == [B.DSA_CHECK_ROWS, 2, 50, 401]
    assert Case(gpu, k_seq_start=[0, -1, 400]).run() == [B.DSA_CHECK_ROWS, 1, 300, -1]
    # a page id equal to the pool size, and a negative one
    c = Case(gpu, paged=True, page_fix=(1, 3, 8))
    assert c.P == 8 and c.run() == [B.DSA_CHECK_PAGE, 1, 3, 8]
    assert Case(gpu, paged=True, page_fix=(0, 1, -1)).run() == [B.DSA_CHECK_PAGE, 0, 1, -1]
    # without a layout the rows and pages are not checked
    assert Case(gpu, k_seq_start=[0, 100, 401]).run(layout=False) == [0, 0, 0, 0]


def test_indices_and_scores(gpu):
    rows = _rows()
    n3 = rows[3][1]
    assert Case(gpu, index_fix=(3, 5, n3)).run() == [B.DSA_CHECK_INDEX, 3, 5, n3]
    assert Case(gpu, index_fix=(0, 70 % K, -2)).run() == [B.DSA_CHECK_INDEX, 0, 70 % K, -2]
    assert Case(gpu, index_fix=(7, 0, rows[7][1] - 1)).run() == [0, 0, 0, 0]   # the last candidate is fine
    assert Case(gpu, score_fix=(4, rows[4][1] - 1)).run() == [B.DSA_CHECK_NAN_SCORE, 4, rows[4][1] - 1, 0]
    assert Case(gpu, score_fix=(4, 5)).run(indices=False) == [B.DSA_CHECK_NAN_SCORE, 4, 5, 0]
    assert Case(gpu, index_fix=(3, 5, n3)).run(indices=False) == [0, 0, 0, 0]


def test_empty_batch_clears_the_report(gpu):
    report = torch.full((4,), 7, dtype=torch.int32, device=gpu)
    bt = B.dsa_batch_t(1, 0, None, None, 0, 0)
    B.dsa_validate(bt, None, None, 0, None, 0, report)
    torch.cuda.synchronize()
    assert report.cpu().tolist() == [0, 0, 0, 0]
