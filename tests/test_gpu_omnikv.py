"""GPU parity of OmniKV: observation-layer token scores and top-b selection
(sp_omnikv_select) against the oracle, the page + token-mask format of the
selection, and a sparse layer's attention over the reused positions of its
own cache (sp_sparse_decode_attn_masked) against the oracle.

Tolerances: a token score is an fp32 sum of D exact bf16 products, so its
error is below about 2^-20 * max|q| * sum_d |k_d| (the bound below); the
largest error observed over these cases is 2.2 % of that bound (1.0e-5
absolute).  Selected sets: equal to the oracle's except candidates within
1e-5 * max(|cutoff|, 1) of the cutoff score; none has differed.  Attention
outputs 2e-3 (bf16 inputs, as for the other attention paths).  The BAND lines
printed under -s record the observed errors and band counts."""
import numpy as np
import pytest
import torch

import kv_cache_selection_sp_amd as sp
import workloads as W
from gpu_util import f64
from oracle import attend, omnikv_select, omnikv_sparse_layer, omnikv_token_scores

pytestmark = pytest.mark.gpu


def _layer(seed, B, Hq, H, D, P, n, hot=0.02):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    G = Hq // H
    dirs = torch.randn(B, H, D, generator=g, device="cuda")
    dirs = dirs / dirs.norm(dim=-1, keepdim=True)
    mark = (torch.rand(B, H, n, generator=g, device="cuda") < hot).float()
    keys = (torch.randn(B, H, n, D, generator=g, device="cuda") + 6 * mark[..., None] * dirs[:, :, None]).to(torch.bfloat16)
    values = torch.randn(B, H, n, D, generator=g, device="cuda").to(torch.bfloat16)
    q = (torch.randn(B, Hq, D, generator=g, device="cuda")
         + 0.5 * D ** 0.5 * dirs.repeat_interleave(G, dim=1)).to(torch.bfloat16)
    max_pages = -(-n // P)
    bt, nblk = W.random_block_table(B, max_pages, g, "cuda")
    kv = sp.PagedKV.allocate(B, Hq, H, D, P, max_pages, nblk, torch.bfloat16, bt)
    sp.sp_build_page_meta(kv, keys.permute(0, 2, 1, 3).contiguous(), values.permute(0, 2, 1, 3).contiguous(),
                          n, None)
    return kv, keys, values, q


def _select(kv, q, top_b):
    B, H = kv.batch, kv.num_kv_heads
    kp = min(top_b, kv.max_pages)
    pages = torch.empty(B, H, kp, dtype=torch.int32, device="cuda")
    mask = torch.empty(B, H, kp, dtype=torch.int32, device="cuda")
    ts = torch.full((B, kv.capacity), -7.0, device="cuda")
    sp.sp_omnikv_select(kv, q, top_b, pages, mask, kp, ts, kv.capacity,
                        sp.workspace(sp.SP_OP_OMNIKV_SELECT, kv, top_b))
    torch.cuda.synchronize()
    return pages, mask, ts, kp


def _positions(pages_row, mask_row, P):
    pos = []
    for p, m in zip(pages_row.tolist(), mask_row.tolist()):
        if p < 0:
            assert m == 0
            continue
        m &= 0xffffffff
        assert m != 0
        pos += [p * P + t for t in range(P) if (m >> t) & 1]
    return pos


@pytest.mark.parametrize("Hq,H,D,P,lens,top_b", [
    (8, 2, 128, 16, [700, 333], 100), (32, 8, 128, 16, [1500, 1499], 256),
    (4, 4, 64, 32, [600, 90], 40), (8, 2, 128, 16, [50, 17], 64),     # L <= b keeps everything
    (8, 2, 128, 16, [50, 17], 100),                                     # b above the capacity (64 slots)
    (32, 2, 128, 16, [900, 517], 128), (24, 2, 64, 32, [800, 777], 77),  # 16 and 12 query heads per KV head
    (128, 8, 128, 16, [300, 45], 33)])                                  # the most query heads
def test_omnikv_select_matches_oracle(Hq, H, D, P, lens, top_b):
    B = 2
    kv, keys, values, q = _layer(3 + top_b, B, Hq, H, D, P, max(lens))
    kv.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
    pages, mask, ts, kp = _select(kv, q, top_b)
    for b in range(B):
        L = lens[b]
        ref = omnikv_token_scores(f64(q[b]), f64(keys[b, :, :L]))
        got = f64(ts[b, :L])
        bound = np.abs(f64(q[b])).max() * np.abs(f64(keys[b, :, :L])).sum(axis=2).max(axis=0) * 1e-6
        e_ = np.abs(got - ref)
        print(f"BAND omnikv score max_abs {float(e_.max()):.3e} max_rel {float((e_ / np.maximum(np.abs(ref), 1e-30)).max()):.3e} "
              f"max_abs_over_bound {float((e_ / bound).max()):.3e}")
        assert bool((np.abs(got - ref) <= bound).all())
        assert bool((ts[b, L:] == -7.0).all())
        pos = _positions(pages[b, 0].cpu(), mask[b, 0].cpu(), P)
        for h in range(1, H):                         # the same selection for every KV head
            assert torch.equal(pages[b, h], pages[b, 0]) and torch.equal(mask[b, h], mask[b, 0])
        pg = [p for p in pages[b, 0].tolist() if p >= 0]
        assert pg == sorted(set(pg))                  # ascending, unique
        want = omnikv_select(ref, top_b)
        assert len(pos) == min(L, top_b) and pos == sorted(pos)
        diff = set(pos) ^ set(want)
        if L > top_b:
            cut_ = np.sort(ref)[::-1][top_b - 1]
            print(f"BAND omnikv select in_1e-5_band {int(np.sum(np.abs(ref - cut_) <= 1e-5 * max(abs(cut_), 1.0)))} "
                  f"diff {len(diff)}")
        if diff:
            cut = np.sort(ref)[::-1][top_b - 1]
            assert all(abs(ref[j] - cut) <= 1e-5 * max(abs(cut), 1.0) for j in diff)


@pytest.mark.parametrize("P,G", [(16, 4), (32, 1)])
def test_sparse_layer_reuses_positions_over_its_own_cache(P, G):
    """Observation layer selects; a second layer (different K/V, same block
    table shape) attends over the same positions."""
    B, H, D, n, top_b = 2, 2, 128, 900, 120
    Hq = G * H
    kv_obs, k1, v1, q1 = _layer(21, B, Hq, H, D, P, n)
    kv_l, k2, v2, q2 = _layer(22, B, Hq, H, D, P, n)
    lens = [900, 477]
    kv_obs.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
    kv_l.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
    pages, mask, _, kp = _select(kv_obs, q1, top_b)
    out = torch.empty(B, Hq, D, device="cuda")
    lse = torch.empty(B, Hq, device="cuda")
    scale = W.default_scale(D)
    sp.sp_sparse_decode_attn_masked(kv_l, q2, pages, mask, kp, scale, out, lse,
                                    sp.workspace(sp.SP_OP_DECODE_ATTN, kv_l, kp))
    torch.cuda.synchronize()
    for b in range(B):
        pos = _positions(pages[b, 0].cpu(), mask[b, 0].cpu(), P)
        o_ref, l_ref = omnikv_sparse_layer(f64(q2[b]), f64(k2[b, :, :lens[b]]), f64(v2[b, :, :lens[b]]), pos,
                                           scale)
        np.testing.assert_allclose(f64(out[b]), o_ref, rtol=0, atol=2e-3)
        np.testing.assert_allclose(f64(lse[b]), l_ref, rtol=0, atol=2e-3)


def test_masked_attention_arbitrary_masks_and_full_masks():
    """Hand-made page lists with random token masks (incl. the partial last
    page and -1 entries) against attention over exactly those slots; full
    masks give the unmasked sparse attention bit for bit."""
    B, Hq, H, D, P, n = 2, 8, 2, 128, 16, 333
    kv, keys, values, q = _layer(31, B, Hq, H, D, P, n)
    k = 6
    g = torch.Generator().manual_seed(5)
    n_pages = -(-n // P)
    sel = torch.stack([torch.stack([torch.randperm(n_pages, generator=g)[:k] for _ in range(H)]) for _ in range(B)])
    sel[0, 1, 2] = -1
    sel[1, 0, 0] = n_pages - 1                       # the partial last page
    msk = torch.randint(0, 1 << 16, (B, H, k), generator=g, dtype=torch.int64)
    msk[:, :, 0] |= 1                                  # every head attends to something
    sel_d = sel.to(torch.int32).cuda()
    msk_d = msk.to(torch.int32).cuda()
    out = torch.empty(B, Hq, D, device="cuda")
    lse = torch.empty(B, Hq, device="cuda")
    scale = W.default_scale(D)
    ws = sp.workspace(sp.SP_OP_DECODE_ATTN, kv, k)
    sp.sp_sparse_decode_attn_masked(kv, q, sel_d, msk_d, k, scale, out, lse, ws)
    torch.cuda.synchronize()
    G = Hq // H
    for b in range(B):
        for h in range(H):
            pos = [int(p) * P + t for p, m in zip(sel[b, h].tolist(), msk[b, h].tolist()) if p >= 0
                   for t in range(P) if (m >> t) & 1 and int(p) * P + t < n]
            for a in range(h * G, (h + 1) * G):
                o, l, _, _ = attend(f64(q[b, a]), f64(keys[b, h, pos]), f64(values[b, h, pos]), scale)
                np.testing.assert_allclose(f64(out[b, a]), o, rtol=0, atol=2e-3)
                assert abs(float(lse[b, a]) - l) <= 2e-3
    full = torch.full_like(msk_d, -1)
    out_m = torch.empty_like(out)
    out_p = torch.empty_like(out)
    sp.sp_sparse_decode_attn_masked(kv, q, sel_d, full, k, scale, out_m, None, ws)
    sp.sp_sparse_decode_attn(kv, q, sel_d, k, scale, out_p, None, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out_m, out_p)
