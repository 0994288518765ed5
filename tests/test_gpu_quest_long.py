"""GPU: Quest selection for long block-table rows.  Up to 5120 pages the
select launch runs the top-k itself (4500 entries: runs of 9 keys over 512
threads); beyond that it only scores; up to
32 768 pages a second launch runs the same top-k with 1024 threads, and
beyond that the list path's threshold search (header, three histogram passes,
counts, list) picks each unit's pages with the sink pages kept as leading
entries and the recent pages as trailing ones.

The same cache seen through a longer block table (the extra entries -1) has
the same pages and the same scores, so both must give the in-launch top-k's
selection bit for bit: over top-k sizes below and above the page count, sink
and recent pages (also filling top_k alone), the maximum over the group,
all-equal scores (ties to the lower page), the fused append, and the
two-launch decode step.  At a real 200 000-token context (12 501 pages) the
selection and the attention over it are checked against the oracle."""
import pytest
import torch

import kv_cache_selection_sp_amd as sp
import workloads as W
from gpu_util import bulk_append, check_quest_unit, new_cache, quest_cache

pytestmark = pytest.mark.gpu

C2 = W.CONFIGS["quest_llama3_8b_b16_ctx32k"]
MID = 4_500     # block-table entries of the long view: the select launch's own top-k, runs of 9
LONG = 12_300   # the 1024-thread top-k
LIST = 33_000   # above 32 * 1024: the list path


def _long_view(kv, n=LONG, seq_lens=None):
    bt = torch.full((kv.batch, n), -1, dtype=torch.int32, device="cuda")
    bt[:, :kv.max_pages] = kv.block_table
    lens = kv.seq_lens.clone() if seq_lens is None else seq_lens
    return sp.PagedKV(kv.k_pool, kv.v_pool, bt, lens, kv.num_q_heads)


def _select(kv, meta, q, top_k, n_sink, n_recent, red):
    sel = torch.full((kv.batch, kv.num_kv_heads, top_k), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((kv.batch, kv.num_kv_heads, kv.max_pages), 3.0, device="cuda")
    sp.sp_select_pages_ex(kv, q, meta, top_k, n_sink, n_recent, red, sel, sc,
                          sp.workspace(sp.SP_OP_SELECT_PAGES, kv, top_k))
    return sel, sc


@pytest.mark.parametrize("n_bt", [MID, LONG, LIST])
@pytest.mark.parametrize("top_k,n_sink,n_recent,red", [
    (24, 0, 0, sp.SP_GROUP_SUM),
    (24, 4, 8, sp.SP_GROUP_SUM),
    (12, 12, 0, sp.SP_GROUP_SUM),     # sink pages fill top_k: nothing left to rank
    (12, 0, 12, sp.SP_GROUP_SUM),     # recent pages fill top_k
    (40, 3, 5, sp.SP_GROUP_MAX),
    (93, 1, 1, sp.SP_GROUP_SUM),      # one page left out
    (200, 2, 2, sp.SP_GROUP_SUM),     # top_k above the page count: every page, -1 padding
])
def test_list_topk_equals_register_topk(top_k, n_sink, n_recent, red, n_bt):
    print(f"long top-k: {n_bt} entries k {top_k} sink {n_sink} recent {n_recent} reduce {red}", flush=True)
    x, kv, meta = quest_cache(C2, 41, 1500, 3)
    kv.seq_lens.copy_(torch.tensor([1500, 777, 0], dtype=torch.int32))   # ragged, one empty sequence
    q = x["q"][0].contiguous()
    sel_a, sc_a = _select(kv, meta, q, top_k, n_sink, n_recent, red)
    kvl = _long_view(kv, n_bt)
    sel_b, sc_b = _select(kvl, meta, q, top_k, n_sink, n_recent, red)
    torch.cuda.synchronize()
    assert torch.equal(sel_a, sel_b)
    assert torch.equal(sc_a, sc_b[:, :, :kv.max_pages])
    assert bool(torch.isneginf(sc_b[:, :, kv.max_pages:]).all())
    assert bool((sel_b[2] == -1).all())
    # the workspace's arrival counters are back at zero (reused by the next call)
    ws = sp.workspace(sp.SP_OP_SELECT_PAGES, kvl, top_k)
    for _ in range(2):
        sel_c = torch.empty_like(sel_b)
        sp.sp_select_pages_ex(kvl, q, meta, top_k, n_sink, n_recent, red, sel_c, None, ws)
        torch.cuda.synchronize()
        assert torch.equal(sel_c, sel_b)
    n_ctr = kv.batch * (kv.num_kv_heads + 1)
    assert int(ws[: 4 * n_ctr].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("n_bt", [MID, LONG, LIST])
@pytest.mark.parametrize("red", [sp.SP_GROUP_SUM, sp.SP_GROUP_MAX])
def test_list_topk_fp32_cache(red, n_bt):
    """fp32 caches (64-dimension heads, the VALU scoring) take the same paths."""
    cfg = W.CONFIGS["quest_f32_b1_h8_d64_ctx1k"]
    x, kv, meta = quest_cache(cfg, 45, 1024, 2)
    q = x["q"][0].contiguous()
    sel_a, sc_a = _select(kv, meta, q, 12, 1, 2, red)
    kvl = _long_view(kv, n_bt)
    sel_b, sc_b = _select(kvl, meta, q, 12, 1, 2, red)
    torch.cuda.synchronize()
    assert torch.equal(sel_a, sel_b)
    assert torch.equal(sc_a, sc_b[:, :, :kv.max_pages])


@pytest.mark.parametrize("n_bt", [MID, LONG, LIST])
def test_list_topk_ties_go_to_lower_pages(n_bt):
    """All keys equal: every page has the same bound, so the lowest unforced
    pages win, beside the forced recent ones."""
    cfg = W.QuestConfig("t", "bf16", batch=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                        context=256, page_size=16, top_k=5, steps=1)
    x = W.quest_inputs(cfg, 70, device="cuda", context=256, batch=1)
    x["keys"][:] = x["keys"][:, :, :1]
    kv = new_cache(1, 8, 2, 128, 16, x["max_pages"], torch.bfloat16, x["block_table"],
                   num_blocks=x["num_blocks"])
    meta = kv.new_meta()
    bulk_append(kv, x["keys"], x["values"], meta)
    kvl = _long_view(kv, n_bt)
    sel, _ = _select(kvl, meta, x["q"][0].contiguous(), 5, 0, 2, sp.SP_GROUP_SUM)
    torch.cuda.synchronize()
    assert sel.cpu().tolist() == [[[0, 1, 2, 14, 15]] * 2]


@pytest.mark.parametrize("n_bt", [LONG, LIST])
def test_list_topk_fused_append_and_two_launch_step(n_bt):
    """sp_append_select_pages and sp_quest_decode_step (two launches above
    12 288 pages) on the long view equal their register-top-k forms on the short
    table: pools, summaries, lengths, selections and scores bit for bit,
    attention to 1e-4 (a different split over workgroups)."""
    x, kv, meta = quest_cache(C2, 43, 3000, 2)
    kv.seq_lens.copy_(torch.tensor([3000, 2100], dtype=torch.int32))
    top_k, n_sink, n_recent, red = 32, 2, 4, sp.SP_GROUP_SUM
    H, Hq, D = kv.num_kv_heads, kv.num_q_heads, kv.head_dim
    scale = W.default_scale(D)
    # the twin: the short table, its own pools
    kv2 = sp.PagedKV(kv.k_pool.clone(), kv.v_pool.clone(), kv.block_table.clone(), kv.seq_lens.clone(),
                     kv.num_q_heads)
    meta2 = meta.clone()
    kvl = _long_view(kv, n_bt)
    assert not sp.sp_quest_step_single_launch(kvl, red) and sp.sp_quest_step_single_launch(kv2, red)
    ws_l = sp.workspace(sp.SP_OP_QUEST_STEP, kvl, top_k)
    ws_s = sp.workspace(sp.SP_OP_QUEST_STEP, kv2, top_k)
    ws_sel = sp.workspace(sp.SP_OP_SELECT_PAGES, kvl, top_k)
    for s in range(3):
        kn, vn, q = x["k_new"][s].contiguous(), x["v_new"][s].contiguous(), x["q"][s].contiguous()
        sel_a = torch.empty(2, H, top_k, dtype=torch.int32, device="cuda")
        sc_a = torch.full((2, H, kvl.max_pages), -5.0, device="cuda")
        out_a = torch.empty(2, Hq, D, device="cuda")
        lse_a = torch.empty(2, Hq, device="cuda")
        if s == 1:
            # the fused append with the list top-k, then the attention
            sp.sp_append_select_pages(kvl, kn, vn, None, None, 0, meta, q, top_k, n_sink, n_recent, red,
                                      sel_a, sc_a, ws_sel)
            sp.sp_sparse_decode_attn(kvl, q, sel_a, top_k, scale, out_a, lse_a,
                                     ws=sp.workspace(sp.SP_OP_DECODE_ATTN, kvl, top_k))
        else:
            sp.sp_quest_decode_step(kvl, kn, vn, None, None, 0, meta, q, top_k, n_sink, n_recent, red, scale,
                                    sel_a, sc_a, out_a, lse_a, ws_l)
        sel_b = torch.empty_like(sel_a)
        sc_b = torch.full((2, H, kv2.max_pages), -5.0, device="cuda")
        out_b = torch.empty_like(out_a)
        lse_b = torch.empty_like(lse_a)
        sp.sp_quest_decode_step(kv2, kn, vn, None, None, 0, meta2, q, top_k, n_sink, n_recent, red, scale,
                                sel_b, sc_b, out_b, lse_b, ws_s)
        torch.cuda.synchronize()
        assert torch.equal(kvl.seq_lens, kv2.seq_lens)
        assert torch.equal(kv.k_pool, kv2.k_pool) and torch.equal(kv.v_pool, kv2.v_pool)
        assert torch.equal(meta, meta2)
        assert torch.equal(sel_a, sel_b)
        assert torch.equal(sc_a[:, :, :kv2.max_pages], sc_b)
        torch.testing.assert_close(out_a, out_b, rtol=0, atol=1e-4)
        torch.testing.assert_close(lse_a, lse_b, rtol=0, atol=1e-4)
    assert sp.sp_quest_step_error(kvl, ws_l) == 0


def test_list_topk_200k_context_matches_oracle():
    """B = 1, 32/8 heads, 200 000 tokens of 16-token pages: 12 501 candidate
    pages after the append, top_k 128 with 4 sink and 32 recent pages.  The
    decode step takes its two launches, the selection the list path; sampled
    KV heads are checked against the oracle (bounds, the top-k set, attention
    over the chosen pages)."""
    context, top_k, n_sink, n_recent = 200_000, 128, 4, 32
    print(f"list top-k at full size: ctx {context} k {top_k}", flush=True)
    x, kv, meta = quest_cache(C2, 47, context, 1)
    assert kv.max_pages > 48 * 256
    H, Hq, D, G = kv.num_kv_heads, kv.num_q_heads, kv.head_dim, C2.group
    scale = W.default_scale(D)
    ws = sp.workspace(sp.SP_OP_QUEST_STEP, kv, top_k)
    for s in range(2):
        sel = torch.empty(1, H, top_k, dtype=torch.int32, device="cuda")
        sc = torch.empty(1, H, kv.max_pages, device="cuda")
        out = torch.empty(1, Hq, D, device="cuda")
        lse = torch.empty(1, Hq, device="cuda")
        sp.sp_quest_decode_step(kv, x["k_new"][s].contiguous(), x["v_new"][s].contiguous(), None, None, 0, meta,
                                x["q"][s].contiguous(), top_k, n_sink, n_recent, sp.SP_GROUP_SUM, scale, sel, sc,
                                out, lse, ws)
        torch.cuda.synchronize()
        assert int(kv.seq_lens[0]) == context + s + 1
        for h in ((0, 5) if s == 0 else (3,)):
            check_quest_unit(x, dict(G=G, P=kv.page_size), 0, h, s, sel[0, h], out[0, h * G:(h + 1) * G],
                             lse[0, h * G:(h + 1) * G], sc[0, h], top_k, scale, torch.bfloat16, n_sink, n_recent)
