"""GPU parity for the Quest variants of the pages' baseline configuration
(Section 5: 16-token pages, 4 sink + 32 recent + 92 selected pages, the first
layers dense) and for max-over-group aggregation of the page bound, against
the oracle under the same comparison rules as the plain Quest tests."""
import numpy as np
import pytest
import torch

import kv_cache_selection_sp_amd as sp
import workloads as W
from gpu_util import TOL, f64, quest_cache, check_selection, score_scale, logical_kv
from oracle import attend, quest_decode_head
from oracle.quest import forced_pages

pytestmark = pytest.mark.gpu

C2 = W.CONFIGS["quest_llama3_8b_b16_ctx32k"]


def _variant_step(cfg, context, batch, top_k, n_sink, n_recent, reduce, Hq=None, seed=11):
    if Hq is not None:
        cfg = W.QuestConfig("v", cfg.dtype, batch, Hq, cfg.num_kv_heads, cfg.head_dim, context,
                            cfg.page_size, top_k, 1)
    x, kv, meta = quest_cache(cfg, seed, context, batch)
    sp.sp_build_page_meta(kv, x["k_new"][0][:, None].contiguous(), x["v_new"][0][:, None].contiguous(), 1, meta)
    B, H, D = kv.batch, kv.num_kv_heads, kv.head_dim
    q = x["q"][0].contiguous()
    sel = torch.empty(B, H, top_k, dtype=torch.int32, device="cuda")
    scores = torch.empty(B, H, kv.max_pages, device="cuda")
    red = sp.SP_GROUP_MAX if reduce == "max" else sp.SP_GROUP_SUM
    sp.sp_select_pages_ex(kv, q, meta, top_k, n_sink, n_recent, red, sel, scores,
                          sp.workspace(sp.SP_OP_SELECT_PAGES, kv, top_k))
    out = torch.empty(B, kv.num_q_heads, D, device="cuda")
    lse = torch.empty(B, kv.num_q_heads, device="cuda")
    scale = W.default_scale(D)
    sp.sp_sparse_decode_attn(kv, q, sel, top_k, scale, out, lse, ws=sp.workspace(sp.SP_OP_DECODE_ATTN, kv, top_k))
    torch.cuda.synchronize()
    return x, kv, q, sel, scores, out, lse, scale


def _check(x, kv, q, sel, scores, out, lse, scale, top_k, n_sink, n_recent, reduce, units):
    G, P = kv.num_q_heads // kv.num_kv_heads, kv.page_size
    dt = kv.dtype
    for (b, h) in units:
        keys, vals = logical_kv(x, b, h, 0)
        qs = f64(q[b, h * G:(h + 1) * G])
        r = quest_decode_head(qs, keys, vals, P, top_k, scale, n_sink, n_recent, reduce)
        N = len(r["scores"])
        # scores of the chosen aggregation, within the fp32 summation error
        err = np.abs(f64(scores[b, h, :N]) - r["scores"])
        assert np.all(err <= 1e-5 * score_scale(qs, r["mins"], r["maxs"]) + 1e-30), err.max()
        row = [int(p) for p in sel[b, h].cpu()]
        forced = forced_pages(N, n_sink, n_recent)
        assert set(forced) <= set(row), "forced pages missing"
        # the other pages follow the top-k rule over the unforced pages
        free = [p for p in range(N) if p not in set(forced)]
        k_free = max(0, min(top_k, N) - len(forced))
        got_free = [p for p in row if p >= 0 and p not in set(forced)]
        assert len(got_free) == k_free
        if 0 < k_free < len(free):
            # the unforced choice, in the index space of the unforced pages
            S = np.asarray(r["scores"])[free]
            mapped = [free.index(p) for p in got_free]
            check_selection(torch.tensor(mapped, dtype=torch.int32), S, k_free)
        assert row == sorted(row[:min(top_k, N)]) + [-1] * (top_k - min(top_k, N))
        # attention over the GPU's own selection
        pages = [p for p in row if p >= 0]
        L = keys.shape[0]
        toks = np.concatenate([np.arange(p * P, min(L, (p + 1) * P)) for p in pages])
        for a in range(G):
            o, l, _, _ = attend(qs[a], f64(keys)[toks], f64(vals)[toks], scale)
            np.testing.assert_allclose(f64(out[b, h * G + a]), o, rtol=0, atol=TOL[dt])
            assert abs(float(lse[b, h * G + a]) - l) <= TOL[dt]


# (3000, 128, 4, 32): the pages' 4 + 32 + 92 budget over 188 pages; then a
# forced-only budget and short sequences where every page is chosen
@pytest.mark.parametrize("context,top_k,n_sink,n_recent", [(3000, 128, 4, 32), (500, 8, 2, 3),
                                                            (500, 5, 0, 5), (100, 16, 4, 12),
                                                            (40, 8, 2, 2)])
def test_sink_and_recent_pages(context, top_k, n_sink, n_recent):
    res = _variant_step(C2, context, 2, top_k, n_sink, n_recent, "sum")
    _check(*res, top_k, n_sink, n_recent, "sum", [(0, 0), (0, 5), (1, 7)])


# G = 1, 4, 8, 16, and the groups the head exchange pads to a power of two
# (slots past G repeat head 0): G = 2, 3, 6, 10, 15
@pytest.mark.parametrize("Hq", [8, 32, 64, 128, 16, 24, 48, 80, 120])
def test_max_over_group(Hq):
    print(f"max over the group: Hq {Hq} Hkv 8", flush=True)
    res = _variant_step(C2, 2000, 2, 32, 0, 0, "max", Hq=Hq)
    _check(*res, 32, 0, 0, "max", [(0, 0), (1, 3), (1, 7)])


@pytest.mark.parametrize("Hq", [32, 48])     # G = 4, 6 with 64-dimension bf16 heads (16 lanes a page)
def test_max_over_group_d64(Hq):
    cfg = W.QuestConfig("d64", "bf16", 2, Hq, 8, 64, 1500, 16, 24, 1)
    res = _variant_step(cfg, 1500, 2, 24, 1, 2, "max", Hq=Hq)
    _check(*res, 24, 1, 2, "max", [(0, 1), (1, 6)])


def test_max_over_group_fp32_sixteen_heads():
    # fp32 data keeps its per-head weights in fp32 (16 heads x 4 channels a lane)
    res = _variant_step(W.CONFIGS["quest_f32_b1_h8_d64_ctx1k"], 1024, 1, 8, 1, 1, "max", Hq=128)
    _check(*res, 8, 1, 1, "max", [(0, 0), (0, 7)])


def test_max_over_group_with_one_head_equals_sum():
    # one head: the same bound, as dot products of packed bf16 pairs (maximum)
    # or fp32 fused multiply-adds (sum), so equal up to the summation
    cfg = W.QuestConfig("g1", "bf16", 2, 8, 8, 128, 1500, 16, 24, 1)
    a = _variant_step(cfg, 1500, 2, 24, 1, 2, "max", seed=5)
    b = _variant_step(cfg, 1500, 2, 24, 1, 2, "sum", seed=5)
    torch.testing.assert_close(a[4], b[4], rtol=1e-6, atol=1e-6)
    assert torch.equal(a[3], b[3])


def test_vortex_configuration_with_fp32_cache():
    cfg = W.CONFIGS["quest_f32_b1_h8_d64_ctx1k"]
    res = _variant_step(cfg, 1024, 1, 8, 1, 2, "sum")
    _check(*res, 8, 1, 2, "sum", [(0, h) for h in range(8)])


def test_dense_attention_over_a_quest_cache():
    """The first layers stay dense: the same cache attended with no selection."""
    x, kv, meta = quest_cache(C2, 21, 900, 2)
    sp.sp_build_page_meta(kv, x["k_new"][0][:, None].contiguous(), x["v_new"][0][:, None].contiguous(), 1, meta)
    q = x["q"][0].contiguous()
    out = torch.empty(2, kv.num_q_heads, kv.head_dim, device="cuda")
    lse = torch.empty(2, kv.num_q_heads, device="cuda")
    scale = W.default_scale(kv.head_dim)
    sp.sp_sparse_decode_attn(kv, q, None, 0, scale, out, lse, ws=sp.workspace(sp.SP_OP_DECODE_ATTN, kv, 0))
    torch.cuda.synchronize()
    G = kv.num_q_heads // kv.num_kv_heads
    for (b, h) in [(0, 0), (1, 6)]:
        keys, vals = logical_kv(x, b, h, 0)
        for a in range(G):
            o, l, _, _ = attend(f64(q[b, h * G + a]), f64(keys), f64(vals), scale)
            np.testing.assert_allclose(f64(out[b, h * G + a]), o, rtol=0, atol=TOL[kv.dtype])
            assert abs(float(lse[b, h * G + a]) - l) <= TOL[kv.dtype]
