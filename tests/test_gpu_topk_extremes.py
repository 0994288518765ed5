"""GPU: the page top-k on score rows built to stress its radix select.

For an fp32 cache with one KV head and one query head, a query that is 1 on
channel 0 and 0 elsewhere gives every page the bound S(p) = M_p0 exactly
(SparseEngine, Appendix A.3 "Quest: Query-Dependent Page Selection": the
bound sums max(q_c m_pc, q_c M_pc) over the channels), so writing the page
summaries sets the score row to chosen fp32 values.  The selection must be
the top_k pages by score with ties to the lower page, in ascending page order,
which a stable host sort gives directly.  Rows: values a few ulps apart,
two clusters sixty orders of magnitude apart, signed zeros and infinities
among normal values, three values only (long runs of ties at the boundary),
and a gap just below the top_k-th page (its bin taken whole).  Page counts
cover the select launch's own top-k (runs of 6 and 9 keys over 512 threads),
the 1024-thread top-k and the list path."""
import numpy as np
import pytest
import torch

import kv_cache_selection_sp_amd as sp

pytestmark = pytest.mark.gpu

D, P = 64, 16


def _scores(kind, n, rng):
    if kind == "ulps":            # 1000 plus 0 .. n-1 ulps, shuffled
        v = (np.full(n, 1000.0, np.float32).view(np.int32) + rng.permutation(n).astype(np.int32)).view(np.float32)
    elif kind == "clusters":      # about half near 1e-30, half near 1e30
        small = rng.random(n) < 0.5
        v = np.where(small, rng.random(n) * 1e-30, 1e30 * (1.0 + rng.random(n))).astype(np.float32)
    elif kind == "signed":        # normal values with +inf, +0 and -0 among them
        v = rng.standard_normal(n).astype(np.float32)
        idx = rng.choice(n, 9, replace=False)
        v[idx[:3]] = np.inf
        v[idx[3:6]] = 0.0
        v[idx[6:]] = -0.0
    elif kind == "ties":          # three values; the boundary falls inside the run of 2.0
        v = rng.choice(np.array([1.0, 2.0, 3.0], np.float32), n, p=[0.5, 0.47, 0.03])
    else:                         # "gap": 64 pages well above the rest
        v = rng.random(n).astype(np.float32)
        v[rng.choice(n, 64, replace=False)] = 5.0 + rng.random(64).astype(np.float32)
    return v


def _expected(v, top_k):
    order = np.lexsort((np.arange(len(v)), -v.astype(np.float64)))   # score desc, page asc; -0.0 == 0.0
    return np.sort(order[:top_k])


@pytest.mark.parametrize("n", [3000, 4600, 9000, 40_000])
@pytest.mark.parametrize("kind,top_k", [("ulps", 100), ("clusters", 300), ("signed", 50), ("ties", 200),
                                        ("gap", 64)])
def test_topk_on_constructed_score_rows(kind, top_k, n):
    print(f"top-k extremes: {kind} n {n} k {top_k}", flush=True)
    rng = np.random.default_rng(n * 7 + len(kind))
    v = _scores(kind, n, rng)
    perm = torch.from_numpy(rng.permutation(n).astype(np.int32))   # scattered blocks
    bt = perm.view(1, n).cuda()
    kv = sp.PagedKV.allocate(1, 1, 1, D, P, n, n, torch.float32, bt, "cuda")
    kv.seq_lens.fill_(n * P)
    meta = kv.new_meta()                                  # [block][head][min, max][D]
    sv = torch.from_numpy(v).cuda()
    blk = bt[0].long()
    meta[blk, 0, 1, 0] = sv                               # maximum of channel 0: the score
    meta[blk, 0, 0, 0] = torch.where(torch.isfinite(sv), sv, torch.zeros_like(sv))   # minimum <= maximum, finite
    q = torch.zeros(1, 1, D, device="cuda")
    q[0, 0, 0] = 1.0
    sel = torch.full((1, 1, top_k), -7, dtype=torch.int32, device="cuda")
    sc = torch.empty(1, 1, n, device="cuda")
    sp.sp_select_pages_ex(kv, q, meta, top_k, 0, 0, sp.SP_GROUP_SUM, sel, sc,
                          sp.workspace(sp.SP_OP_SELECT_PAGES, kv, top_k))
    torch.cuda.synchronize()
    got_scores = sc[0, 0].cpu().numpy()
    finite = np.isfinite(v)
    assert np.array_equal(got_scores[finite], v[finite]) and np.all(np.isposinf(got_scores[~finite]))
    assert sel[0, 0].cpu().numpy().tolist() == _expected(v, top_k).tolist()
