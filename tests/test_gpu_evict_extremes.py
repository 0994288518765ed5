"""GPU: H2O eviction on score rows built to stress its threshold search.

sp_h2o_evict_compact keeps the last recent_window slots and, of the others,
the budget - recent_window with the largest scores, ties to the lower slot
(SparseEngine, Appendix A.3 "H2O: Accumulated Scores and Online Eviction",
with the tie reading of lower positions first), and compacts them in slot
order.  Scores are written directly; the expected kept slots come from a
stable host sort.  Rows: values a few ulps apart, clusters sixty orders of
magnitude apart, signed zeros and infinities, three values only, a gap at
the boundary, and the steady-state case of one slot over the budget; slot
capacities up to 8192 (one workgroup per unit) and above (the list path)."""
import numpy as np
import pytest
import torch

import kv_cache_selection_sp_amd as sp

pytestmark = pytest.mark.gpu

D, P, H = 64, 16, 2


def _scores(kind, n, rng):
    if kind == "ulps":
        return (np.full(n, 3.5, np.float32).view(np.int32) + rng.permutation(n).astype(np.int32)).view(np.float32)
    if kind == "clusters":
        small = rng.random(n) < 0.5
        return np.where(small, rng.random(n) * 1e-30, 1e30 * (1.0 + rng.random(n))).astype(np.float32)
    if kind == "signed":
        v = rng.standard_normal(n).astype(np.float32)
        idx = rng.choice(n, 9, replace=False)
        v[idx[:3]] = np.inf
        v[idx[3:6]] = 0.0
        v[idx[6:]] = -0.0
        return v
    if kind == "ties":
        return rng.choice(np.array([1.0, 2.0, 3.0], np.float32), n, p=[0.3, 0.6, 0.1])
    v = rng.random(n).astype(np.float32)             # "gap"
    v[: n // 2] += 10.0
    return v


def _kept(v, L, budget, window):
    cand = np.arange(L - window)
    order = np.lexsort((cand, -v[:L - window].astype(np.float64)))   # score desc, slot asc; -0.0 == 0.0
    keep = np.sort(order[:budget - window])
    return np.concatenate([keep, np.arange(L - window, L)])


@pytest.mark.parametrize("cap,budget,window", [(1200, 1024, 128), (1025, 1024, 128), (9000, 8192, 128),
                                               (40_000, 8192, 32)])
@pytest.mark.parametrize("kind", ["ulps", "clusters", "signed", "ties", "gap"])
def test_evict_on_constructed_scores(kind, cap, budget, window):
    print(f"evict extremes: {kind} cap {cap} budget {budget} window {window}", flush=True)
    rng = np.random.default_rng(cap + len(kind))
    n_pages = cap // P + 1
    bt = torch.from_numpy(rng.permutation(n_pages).astype(np.int32)).view(1, n_pages)
    kv = sp.PagedKV.allocate(1, H, H, D, P, n_pages, n_pages, torch.float32, bt, "cuda")
    slot_cap = kv.capacity
    L = cap
    kv.seq_lens.fill_(L)
    rows = [_scores(kind, slot_cap, rng) for _ in range(H)]
    scores = torch.from_numpy(np.stack(rows)).view(1, H, slot_cap).cuda()
    slot_pos = torch.arange(slot_cap, dtype=torch.int32, device="cuda").view(1, 1, slot_cap).repeat(1, H, 1)
    sp.sp_h2o_evict_compact(kv, scores, slot_pos, slot_cap, budget, window,
                            sp.workspace(sp.SP_OP_H2O_EVICT, kv, budget))
    torch.cuda.synchronize()
    assert int(kv.seq_lens[0]) == budget
    for h in range(H):
        keep = _kept(rows[h], L, budget, window)
        assert slot_pos[0, h, :budget].cpu().numpy().tolist() == keep.tolist()
        got = scores[0, h, :budget].cpu().numpy()
        assert np.array_equal(got, rows[h][keep])
