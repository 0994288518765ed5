"""GPU: the fused Quest decode step (sp_quest_decode_step: the decode append,
the page selection and the sparse attention in one launch) against
sp_append_select_pages followed by sp_sparse_decode_attn on a twin cache.
Pools, page summaries, slot positions, lengths, selections and page scores
must be equal bit for bit; out and lse agree to 1e-4 (the attention is split
over workgroups differently, so only the fp32 summation order differs) and
are checked against the oracle on sampled units.  Several steps run on one
workspace: its arrival counters return to zero and the error word stays 0
(the per-unit epochs count up, so no flag needs resetting).  Covered: the
single launch (up to 12 288 pages: top-k runs of 8, 16 and 24 keys per thread
over 512 threads; selections staged in LDS up to 2048 pages and written
directly above)
with the sum over the group for bf16 with G in {4, 8}, P in {16, 32}, fp32
with G = 1 (the VALU engine), and with the maximum over the group for bf16;
ragged, empty and fully-selected sequences, forced sink and recent pages, no
append; and the two-launch path the call takes otherwise (the maximum in
fp32, more than 12 288 pages).  Every case first checks which of the two forms
sp_quest_step_single_launch reports."""
import pytest
import torch

import kv_cache_selection_sp_amd as sp
import workloads as W
from gpu_util import check_quest_unit, quest_cache

pytestmark = pytest.mark.gpu

C1 = W.CONFIGS["quest_f32_b1_h8_d64_ctx1k"]
C2 = W.CONFIGS["quest_llama3_8b_b16_ctx32k"]
C5 = W.CONFIGS["quest_gqa8_b4_ctx128k"]
C16 = W.QuestConfig("quest_g16", "bf16", 2, 128, 8, 128, 2000, 16, 16, 3)   # 16 query heads per KV head
C6 = W.QuestConfig("quest_g6", "bf16", 2, 48, 8, 128, 2000, 16, 16, 3)      # 6 (a padded head exchange)


def _twin(kv, meta):
    kv2 = sp.PagedKV(kv.k_pool.clone(), kv.v_pool.clone(), kv.block_table.clone(), kv.seq_lens.clone(),
                     kv.num_q_heads)
    return kv2, meta.clone()


def _run(cfg, context, batch, top_k, n_sink, n_recent, red, lens, steps, append=True, oracle_units=(), single=True):
    # the oracle check covers the sum aggregation (the max form is checked against the oracle elsewhere)
    if red != sp.SP_GROUP_SUM:
        oracle_units = ()
    print(f"quest step: {cfg.name} ctx {context} B {batch} k {top_k} sink {n_sink} recent {n_recent} "
          f"reduce {red} lens {lens} append {append}", flush=True)
    x, kv, meta = quest_cache(cfg, 31, context, batch)
    if lens is not None:
        kv.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
    kv2, meta2 = _twin(kv, meta)
    assert sp.sp_quest_step_single_launch(kv, red) == single, f"{kv.max_pages} pages, reduce {red}"
    B, H, Hq, D = batch, cfg.num_kv_heads, cfg.num_q_heads, cfg.head_dim
    cap = kv.capacity
    scale = W.default_scale(D)
    slot_a = torch.full((B, H, cap), -3, dtype=torch.int32, device="cuda")
    slot_b = slot_a.clone()
    pos_new = (kv.seq_lens + 1000).contiguous()
    ws = sp.workspace(sp.SP_OP_QUEST_STEP, kv, top_k)
    ws_sel = sp.workspace(sp.SP_OP_SELECT_PAGES, kv2, top_k)
    ws_att = sp.workspace(sp.SP_OP_DECODE_ATTN, kv2, top_k)
    for s in range(min(steps, cfg.steps)):
        kn = x["k_new"][s].contiguous() if append else None
        vn = x["v_new"][s].contiguous() if append else None
        q = x["q"][s].contiguous()
        sel_a = torch.empty(B, H, top_k, dtype=torch.int32, device="cuda")
        sc_a = torch.full((B, H, kv.max_pages), -5.0, device="cuda")
        out_a = torch.full((B, Hq, D), float("nan"), device="cuda")
        lse_a = torch.full((B, Hq), float("nan"), device="cuda")
        sp.sp_quest_decode_step(kv, kn, vn, pos_new if append else None, slot_a if append else None, cap, meta,
                                q, top_k, n_sink, n_recent, red, scale, sel_a, sc_a, out_a, lse_a, ws)
        sel_b = torch.empty_like(sel_a)
        sc_b = torch.full_like(sc_a, -5.0)
        out_b = torch.empty_like(out_a)
        lse_b = torch.empty_like(lse_a)
        if append:
            sp.sp_append_select_pages(kv2, kn, vn, pos_new, slot_b, cap, meta2, q, top_k, n_sink, n_recent, red,
                                      sel_b, sc_b, ws_sel)
        else:
            sp.sp_select_pages_ex(kv2, q, meta2, top_k, n_sink, n_recent, red, sel_b, sc_b, ws_sel)
        sp.sp_sparse_decode_attn(kv2, q, sel_b, top_k, scale, out_b, lse_b, ws=ws_att)
        torch.cuda.synchronize()
        assert torch.equal(kv.seq_lens, kv2.seq_lens)
        assert torch.equal(kv.k_pool, kv2.k_pool) and torch.equal(kv.v_pool, kv2.v_pool)
        assert torch.equal(meta, meta2)
        assert torch.equal(slot_a, slot_b)
        assert torch.equal(sel_a, sel_b)
        assert torch.equal(sc_a, sc_b)
        assert torch.isfinite(out_a).all()
        torch.testing.assert_close(out_a, out_b, rtol=0, atol=1e-4)
        torch.testing.assert_close(lse_a, lse_b, rtol=0, atol=1e-4, equal_nan=False)
        # the selection's arrival counters (per unit, then per sequence) back at zero, error word 0
        head = ws[: 4 * (B * H + B)].view(torch.int32)
        assert int(head.abs().sum()) == 0, "select counters not zero"
        assert sp.sp_quest_step_error(kv, ws) == 0
        for (b, h) in oracle_units:
            # the oracle replays the workload's tokens: units of sequences at their full context
            if append and (lens is None or lens[b] == context):
                G = cfg.group
                check_quest_unit(x, dict(G=G, P=cfg.page_size), b, h, s, sel_a[b, h],
                                 out_a[b, h * G:(h + 1) * G], lse_a[b, h * G:(h + 1) * G], sc_a[b, h], top_k,
                                 scale, W.torch_dtype(cfg.dtype), n_sink, n_recent)
        if append:
            pos_new += 1


@pytest.mark.parametrize("cfg,context,batch,top_k,n_sink,n_recent,red,lens,units", [
    (C2, 2000, 2, 16, 0, 0, sp.SP_GROUP_SUM, None, [(0, 0), (1, 7)]),       # a fresh page first
    (C2, 2000, 3, 16, 1, 2, sp.SP_GROUP_SUM, [2000, 1963, 0], [(0, 3)]),   # ragged, one empty sequence
    (C1, 1000, 1, 8, 0, 0, sp.SP_GROUP_SUM, None, [(0, 0), (0, 5)]),        # fp32, D 64, G 1 (VALU engine)
    (C5, 3000, 2, 24, 0, 0, sp.SP_GROUP_SUM, [3000, 2017], [(0, 2)]),       # G 8, P 32
    (C2, 100, 2, 16, 0, 0, sp.SP_GROUP_SUM, None, [(0, 1)]),               # top_k >= pages: all selected
    (C2, 40000, 1, 128, 4, 32, sp.SP_GROUP_SUM, None, [(0, 6)]),          # 2501 pages, sink + recent
    (C2, 70000, 1, 64, 0, 3, sp.SP_GROUP_SUM, None, [(0, 1)]),            # 4376 pages: runs of 16 keys
    (C2, 150000, 1, 64, 2, 3, sp.SP_GROUP_SUM, None, [(0, 1)]),           # 9376 pages: runs of 24 keys
    (C2, 30000, 1, 1100, 0, 0, sp.SP_GROUP_SUM, None, [(0, 2)]),          # top_k > 1024
    (C2, 40000, 1, 2100, 2, 2, sp.SP_GROUP_SUM, None, [(0, 4)]),          # top_k > 2048: unstaged output
    (C5, 3000, 2, 24, 0, 0, sp.SP_GROUP_MAX, [3000, 2017], []),          # max over the group (bf16, D 128)
    (C2, 2000, 2, 16, 1, 2, sp.SP_GROUP_MAX, None, []),                  # max over the group, sink + recent
    (C16, 2000, 2, 16, 0, 0, sp.SP_GROUP_SUM, None, [(1, 6)]),             # G 16
    (C16, 2000, 2, 16, 1, 2, sp.SP_GROUP_MAX, None, []),                 # max over 16 heads
    (C6, 2000, 2, 16, 0, 1, sp.SP_GROUP_MAX, None, []),                  # max over 6 heads
    (C6, 2000, 2, 16, 0, 0, sp.SP_GROUP_SUM, None, [(1, 2)]),             # G 6, the sum
])
def test_single_launch_equals_two_launches(cfg, context, batch, top_k, n_sink, n_recent, red, lens, units):
    _run(cfg, context, batch, top_k, n_sink, n_recent, red, lens, steps=3, oracle_units=units)


def test_without_append():
    _run(C2, 3000, 2, 32, 0, 0, sp.SP_GROUP_SUM, None, steps=2, append=False)


@pytest.mark.parametrize("cfg,context,batch,top_k,red", [
    (C1, 1000, 1, 8, sp.SP_GROUP_MAX),      # max over the group in fp32: two launches
    (C2, 200000, 1, 64, sp.SP_GROUP_SUM),   # 12 501 pages: two launches
])
def test_two_launch_path(cfg, context, batch, top_k, red):
    _run(cfg, context, batch, top_k, 0, 0, red, None, steps=2, oracle_units=[(0, 1)], single=False)
