"""GPU: the fused decode step front (sp_append_select_pages: one token
appended to every sequence, then the Quest selection, in one launch) equals
sp_build_page_meta with one token followed by sp_select_pages_ex, bit for bit:
pools, page summaries, slot positions, lengths, selections and page scores.
Covered: several steps in a row on one workspace (its counters return to
zero), a token opening a fresh page and folding into a partial one, the token's
page in a later chunk of a long sequence, ragged, empty and full sequences, an
invalid block id under the token's page, both group aggregations with forced
sink and recent pages, bf16 and fp32, D in {64, 128}, P in {16, 32}.  One step
is also checked against the oracle."""
import pytest
import torch

import kv_cache_selection_sp_amd as sp
import workloads as W
from gpu_util import check_quest_unit, quest_cache

pytestmark = pytest.mark.gpu

C1 = W.CONFIGS["quest_f32_b1_h8_d64_ctx1k"]
C2 = W.CONFIGS["quest_llama3_8b_b16_ctx32k"]
C5 = W.CONFIGS["quest_gqa8_b4_ctx128k"]


def _twin(kv, meta):
    """An independent copy of the cache state (same block table)."""
    kv2 = sp.PagedKV(kv.k_pool.clone(), kv.v_pool.clone(), kv.block_table.clone(), kv.seq_lens.clone(),
                     kv.num_q_heads)
    return kv2, meta.clone()


def _state_equal(kv_a, meta_a, kv_b, meta_b):
    assert torch.equal(kv_a.seq_lens, kv_b.seq_lens)
    assert torch.equal(kv_a.k_pool, kv_b.k_pool)
    assert torch.equal(kv_a.v_pool, kv_b.v_pool)
    assert torch.equal(meta_a, meta_b)


@pytest.mark.parametrize("cfg,context,batch,top_k,n_sink,n_recent,red,lens", [
    (C2, 2000, 2, 16, 0, 0, sp.SP_GROUP_SUM, None),            # 2000 % 16 == 0: a fresh page first
    (C2, 2000, 3, 16, 1, 2, sp.SP_GROUP_SUM, [2000, 1963, 0]),  # ragged, one empty sequence
    (C1, 1000, 1, 8, 0, 0, sp.SP_GROUP_SUM, None),             # fp32, D 64, G 1
    (C5, 3000, 2, 24, 2, 3, sp.SP_GROUP_MAX, [3000, 2017]),     # G 8, P 32, max over the group
    (C2, 40000, 1, 128, 4, 32, sp.SP_GROUP_SUM, None),         # > 1024 pages: the token in a late chunk
])
def test_fused_equals_append_then_select(cfg, context, batch, top_k, n_sink, n_recent, red, lens):
    x, kv, meta = quest_cache(cfg, 31, context, batch)
    if lens is not None:
        kv.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
    kv2, meta2 = _twin(kv, meta)
    B, H = batch, cfg.num_kv_heads
    cap = kv.capacity
    slot_a = torch.full((B, H, cap), -3, dtype=torch.int32, device="cuda")
    slot_b = slot_a.clone()
    pos_new = (kv.seq_lens + 1000).contiguous()
    ws_a = sp.workspace(sp.SP_OP_SELECT_PAGES, kv, top_k)
    for s in range(min(3, cfg.steps)):
        kn = x["k_new"][s].contiguous()                 # [B][H_kv][D]
        vn = x["v_new"][s].contiguous()
        q = x["q"][s].contiguous()
        sel_a = torch.empty(B, H, top_k, dtype=torch.int32, device="cuda")
        sc_a = torch.full((B, H, kv.max_pages), -5.0, device="cuda")
        sp.sp_append_select_pages(kv, kn, vn, pos_new, slot_a, cap, meta, q, top_k, n_sink, n_recent, red,
                                  sel_a, sc_a, ws_a)
        sp.sp_build_page_meta(kv2, kn[:, None].contiguous(), vn[:, None].contiguous(), 1, meta2, pos_new,
                              slot_b, cap)
        sel_b = torch.empty_like(sel_a)
        sc_b = torch.full_like(sc_a, -5.0)
        sp.sp_select_pages_ex(kv2, q, meta2, top_k, n_sink, n_recent, red, sel_b, sc_b,
                              sp.workspace(sp.SP_OP_SELECT_PAGES, kv2, top_k))
        torch.cuda.synchronize()
        _state_equal(kv, meta, kv2, meta2)
        assert torch.equal(slot_a, slot_b)
        assert torch.equal(sel_a, sel_b)
        assert torch.equal(sc_a, sc_b)
        pos_new += 1
    # every counter, the per-sequence ones included, is back at zero
    n = B * H + B
    assert int(ws_a[: 4 * n].view(torch.int32).abs().sum()) == 0


def test_full_sequence_and_invalid_block():
    """A sequence at capacity takes no token (length unchanged); a token whose
    page has an invalid block id writes no pool or summary entry (the page
    scores -inf) but still counts, as with the separate append."""
    cfg = C2
    x, kv, meta = quest_cache(cfg, 41, 700, 3)
    cap = kv.capacity
    kv.seq_lens.copy_(torch.tensor([cap, 700, 650], dtype=torch.int32))
    kv.block_table[1, 700 // 16] = -1
    kv.block_table[2, 650 // 16] = kv.num_blocks + 5
    kv2, meta2 = _twin(kv, meta)
    top_k = 8
    kn, vn, q = x["k_new"][0].contiguous(), x["v_new"][0].contiguous(), x["q"][0].contiguous()
    sel_a = torch.empty(3, 8, top_k, dtype=torch.int32, device="cuda")
    sc_a = torch.empty(3, 8, kv.max_pages, device="cuda")
    sp.sp_append_select_pages(kv, kn, vn, None, None, 0, meta, q, top_k, 0, 0, sp.SP_GROUP_SUM, sel_a, sc_a,
                              sp.workspace(sp.SP_OP_SELECT_PAGES, kv, top_k))
    sp.sp_build_page_meta(kv2, kn[:, None].contiguous(), vn[:, None].contiguous(), 1, meta2)
    sel_b, sc_b = torch.empty_like(sel_a), torch.empty_like(sc_a)
    sp.sp_select_pages_ex(kv2, q, meta2, top_k, 0, 0, sp.SP_GROUP_SUM, sel_b, sc_b,
                          sp.workspace(sp.SP_OP_SELECT_PAGES, kv2, top_k))
    torch.cuda.synchronize()
    assert kv.seq_lens.tolist() == [cap, 701, 651]
    _state_equal(kv, meta, kv2, meta2)
    assert torch.equal(sel_a, sel_b)
    n_pages = [cap // 16, 701 // 16 + 1, 651 // 16 + 1]
    for b in range(3):
        assert torch.equal(sc_a[b, :, :n_pages[b]], sc_b[b, :, :n_pages[b]])
    assert bool(torch.isinf(sc_a[1, :, 700 // 16]).all()) and bool(torch.isinf(sc_a[2, :, 650 // 16]).all())


@pytest.mark.parametrize("cfg,context,batch,top_k", [(C2, 2000, 2, 16), (C5, 3000, 1, 24)])
def test_fused_step_matches_oracle(cfg, context, batch, top_k):
    x, kv, meta = quest_cache(cfg, 21, context, batch)
    scale = W.default_scale(cfg.head_dim)
    dtype = W.torch_dtype(cfg.dtype)
    B, H, G, D = batch, cfg.num_kv_heads, cfg.group, cfg.head_dim
    ws = sp.workspace(sp.SP_OP_SELECT_PAGES, kv, top_k)
    ws_att = sp.workspace(sp.SP_OP_DECODE_ATTN, kv, top_k)
    for s in range(2):
        q = x["q"][s].contiguous()
        sel = torch.empty(B, H, top_k, dtype=torch.int32, device="cuda")
        scores = torch.empty(B, H, kv.max_pages, device="cuda")
        sp.sp_append_select_pages(kv, x["k_new"][s].contiguous(), x["v_new"][s].contiguous(), None, None, 0,
                                  meta, q, top_k, 0, 0, sp.SP_GROUP_SUM, sel, scores, ws)
        out = torch.empty(B, cfg.num_q_heads, D, device="cuda")
        lse = torch.empty(B, cfg.num_q_heads, device="cuda")
        sp.sp_sparse_decode_attn(kv, q, sel, top_k, scale, out, lse, ws=ws_att)
        torch.cuda.synchronize()
        for b in range(B):
            for h in range(H):
                check_quest_unit(x, dict(G=G, P=cfg.page_size), b, h, s, sel[b, h], out[b, h * G:(h + 1) * G],
                                 lse[b, h * G:(h + 1) * G], scores[b, h], top_k, scale, dtype)
