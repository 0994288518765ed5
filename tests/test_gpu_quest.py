"""GPU parity: page summaries (bit-exact), bound scores, top-k sets and sparse
attention against the oracle, on reduced and edge-case shapes."""
import math

import numpy as np
import pytest
import torch

import kv_cache_selection_sp_amd as sp
import workloads as W
from gpu_util import (TOL, f64, new_cache, bulk_append, quest_cache, quest_gpu_step,
                      check_quest_unit, check_selection, logical_kv)
from oracle import page_extrema, quest_decode_head, attend

pytestmark = pytest.mark.gpu

C1 = W.CONFIGS["quest_f32_b1_h8_d64_ctx1k"]
C2 = W.CONFIGS["quest_llama3_8b_b16_ctx32k"]
C5 = W.CONFIGS["quest_gqa8_b4_ctx128k"]


def _cfg(kv):
    return dict(G=kv.num_q_heads // kv.num_kv_heads, P=kv.page_size)


@pytest.mark.parametrize("cfg,context,batch", [(C1, 1000, 1), (C2, 531, 2), (C5, 700, 1)])
def test_page_summaries_bit_exact_and_rebuild_equal(cfg, context, batch):
    x, kv, meta = quest_cache(cfg, 11, context, batch)
    P = cfg.page_size
    n_pages = -(-context // P)
    for b in range(batch):
        for h in range(cfg.num_kv_heads):
            mins, maxs = page_extrema(x["keys"][b, h].cpu(), P)
            gm, gM = sp.read_meta(kv, meta, b, h, n_pages)
            assert np.array_equal(f64(gm), mins) and np.array_equal(f64(gM), maxs)
    # rebuild from the pool equals the incremental fold bit for bit
    meta2 = torch.full_like(meta, 7)
    sp.sp_build_page_meta(kv, None, None, 0, meta2)
    torch.cuda.synchronize()
    for b in range(batch):
        blocks = kv.block_table[b, :n_pages].long()
        assert torch.equal(meta[blocks], meta2[blocks])
    # the pool holds the logical tokens
    kk, vv = sp.read_slots(kv, 0, 1, context)
    assert torch.equal(kk, x["keys"][0, 1]) and torch.equal(vv, x["values"][0, 1])
    assert int(kv.seq_lens[0]) == context


def test_incremental_fold_across_page_boundaries():
    """Tokens appended one at a time and in odd-sized chunks give the same
    summaries as the rebuild (pages start fresh at offset 0)."""
    cfg = C2
    x = W.quest_inputs(cfg, 3, device="cuda", context=112, batch=2)
    kv = new_cache(2, 32, 8, 128, 16, x["max_pages"], torch.bfloat16, x["block_table"],
                   num_blocks=x["num_blocks"])
    meta = kv.new_meta()
    keys, vals = x["keys"], x["values"]
    for lo, hi in [(0, 1), (1, 16), (16, 17), (17, 40), (40, 41), (41, 77), (77, 90), (90, 96),
                   (96, 112)]:
        bulk_append(kv, keys[:, :, lo:hi], vals[:, :, lo:hi], meta)
    meta2 = kv.new_meta()
    sp.sp_build_page_meta(kv, None, None, 0, meta2)
    torch.cuda.synchronize()
    assert torch.equal(meta, meta2)
    for h in range(8):
        mins, maxs = page_extrema(keys[1, h].cpu(), 16)
        gm, gM = sp.read_meta(kv, meta, 1, h, 7)
        assert np.array_equal(f64(gm), mins) and np.array_equal(f64(gM), maxs)
    # the pool holds every appended token and the lengths advanced exactly
    assert kv.seq_lens.cpu().tolist() == [112, 112]
    for b in range(2):
        kk, vv = sp.read_slots(kv, b, 5, 112)
        assert torch.equal(kk, keys[b, 5]) and torch.equal(vv, vals[b, 5])


@pytest.mark.parametrize("cfg,context,batch,top_k", [
    (C1, 1024, 1, 8),          # the parity-sized fp32 workload at full size
    (C2, 2000, 2, 16),         # GQA 4, several splits and a ragged last page
    (C2, 300, 2, 64),          # top_k >= pages: all pages, -1 padding
    (C5, 3000, 2, 24),         # GQA 8, 32-token pages
    (C2, 40000, 1, 128),       # > 1024 candidate pages: multi-chunk top-k scan
    (C2, 40000, 1, 1500),      # top_k > 1024
    (C2, 40000, 1, 2100),      # top_k > 2048: the selection is written without LDS staging
])
def test_quest_step_matches_oracle(cfg, context, batch, top_k):
    x, kv, meta = quest_cache(cfg, 21, context, batch)
    scale = W.default_scale(cfg.head_dim)
    dtype = W.torch_dtype(cfg.dtype)
    for s in range(min(2, cfg.steps)):
        sel, scores, out, lse = quest_gpu_step(kv, meta, x, s, top_k, scale)
        torch.cuda.synchronize()
        G = cfg.group
        for b in range(batch):
            for h in range(cfg.num_kv_heads):
                check_quest_unit(x, _cfg(kv), b, h, s, sel[b, h], out[b, h * G:(h + 1) * G],
                                 lse[b, h * G:(h + 1) * G], scores[b, h], top_k, scale, dtype)


def test_select_without_page_scores_uses_workspace():
    x, kv, meta = quest_cache(C2, 5, 900, 2)
    scale = W.default_scale(128)
    sel_a, _, out_a, _ = quest_gpu_step(kv, meta, x, 0, 16, scale, with_scores=True)
    # same state: rerun selection with the workspace path on a fresh cache
    x2, kv2, meta2 = quest_cache(C2, 5, 900, 2)
    sel_b, _, out_b, _ = quest_gpu_step(kv2, meta2, x2, 0, 16, scale, with_scores=False)
    torch.cuda.synchronize()
    assert torch.equal(sel_a, sel_b) and torch.equal(out_a, out_b)


def test_deterministic_repeat():
    x, kv, meta = quest_cache(C5, 8, 2500, 1)
    scale = W.default_scale(128)
    sel, _, out, lse = quest_gpu_step(kv, meta, x, 0, 32, scale)
    ws = sp.workspace(sp.SP_OP_DECODE_ATTN, kv, 32)
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    sp.sp_sparse_decode_attn(kv, x["q"][0].contiguous(), sel, 32, scale, out2, lse2, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("context", [1, 5, 16, 17])
def test_short_sequences(context):
    """Fewer tokens than one page, exactly one page, one page plus one."""
    x, kv, meta = quest_cache(C2, 31, context, 2)
    scale = W.default_scale(128)
    sel, scores, out, lse = quest_gpu_step(kv, meta, x, 0, 4, scale)
    torch.cuda.synchronize()
    for b in range(2):
        for h in range(8):
            check_quest_unit(x, _cfg(kv), b, h, 0, sel[b, h], out[b, 4 * h:4 * h + 4],
                             lse[b, 4 * h:4 * h + 4], scores[b, h], 4, scale, torch.bfloat16)


def test_hand_written_selection_with_holes_and_empty_sequence():
    """Explicit page lists with -1 entries and out-of-range pages are skipped;
    a sequence with no tokens returns zeros and lse = -inf."""
    x, kv, meta = quest_cache(C2, 41, 200, 2)
    kv.seq_lens[1] = 0
    sel = torch.tensor([[[3, -1, 0, 9999], [-1, -1, -1, 12]] + [[0, 1, 2, 3]] * 6,
                        [[0, 1, 2, 3]] * 8], dtype=torch.int32, device="cuda")
    q = x["q"][0].contiguous()
    out = torch.empty(2, 32, 128, device="cuda")
    lse = torch.empty(2, 32, device="cuda")
    ws = sp.workspace(sp.SP_OP_DECODE_ATTN, kv, 4)
    scale = W.default_scale(128)
    sp.sp_sparse_decode_attn(kv, q, sel, 4, scale, out, lse, ws=ws)
    torch.cuda.synchronize()
    keys, vals = f64(x["keys"][0]), f64(x["values"][0])
    for h, pages in [(0, [3, 0]), (1, [12]), (2, [0, 1, 2, 3])]:
        toks = np.concatenate([np.arange(p * 16, min(200, p * 16 + 16)) for p in sorted(pages)])
        for a in range(4):
            o, l, _, _ = attend(f64(q[0, 4 * h + a]), keys[h][toks], vals[h][toks], scale)
            np.testing.assert_allclose(f64(out[0, 4 * h + a]), o, atol=2e-3)
    assert bool((out[1] == 0).all()) and bool(torch.isneginf(lse[1]).all())


def test_fp32_mha_matches_oracle_tightly():
    """fp32, G = 1 (the VALU path) at the 1e-5 bar, with head_dim 128."""
    cfg = W.QuestConfig("t", "f32", batch=2, num_q_heads=4, num_kv_heads=4, head_dim=128,
                        context=500, page_size=32, top_k=5, steps=1)
    x, kv, meta = quest_cache(cfg, 51, 500, 2)
    scale = W.default_scale(128)
    sel, scores, out, lse = quest_gpu_step(kv, meta, x, 0, 5, scale)
    torch.cuda.synchronize()
    for b in range(2):
        for h in range(4):
            check_quest_unit(x, _cfg(kv), b, h, 0, sel[b, h], out[b, h:h + 1], lse[b, h:h + 1],
                             scores[b, h], 5, scale, torch.float32)


def test_bf16_mha_valu_path_and_head_dim_64():
    cfg = W.QuestConfig("t", "bf16", batch=1, num_q_heads=4, num_kv_heads=4, head_dim=64,
                        context=333, page_size=16, top_k=6, steps=1)
    x, kv, meta = quest_cache(cfg, 52, 333, 1)
    scale = W.default_scale(64)
    sel, scores, out, lse = quest_gpu_step(kv, meta, x, 0, 6, scale)
    torch.cuda.synchronize()
    for h in range(4):
        check_quest_unit(x, _cfg(kv), 0, h, 0, sel[0, h], out[0, h:h + 1], lse[0, h:h + 1],
                         scores[0, h], 6, scale, torch.bfloat16)


@pytest.mark.parametrize("D,P,G", [(64, 16, 2), (64, 32, 16), (128, 32, 4)])
def test_mfma_path_other_shapes(D, P, G):
    cfg = W.QuestConfig("t", "bf16", batch=2, num_q_heads=2 * G, num_kv_heads=2, head_dim=D,
                        context=450, page_size=P, top_k=7, steps=1)
    x, kv, meta = quest_cache(cfg, 60 + D + P + G, 450, 2)
    scale = W.default_scale(D)
    sel, scores, out, lse = quest_gpu_step(kv, meta, x, 0, 7, scale)
    torch.cuda.synchronize()
    for b in range(2):
        for h in range(2):
            check_quest_unit(x, _cfg(kv), b, h, 0, sel[b, h], out[b, h * G:(h + 1) * G],
                             lse[b, h * G:(h + 1) * G], scores[b, h], 7, scale, torch.bfloat16)


def test_ties_go_to_lower_pages():
    """All keys equal: every page has the same bound, so the lowest pages win."""
    cfg = W.QuestConfig("t", "bf16", batch=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                        context=256, page_size=16, top_k=5, steps=1)
    x = W.quest_inputs(cfg, 70, device="cuda", context=256, batch=1)
    x["keys"][:] = x["keys"][:, :, :1]
    x["k_new"][:] = x["keys"][:, :, 0]
    kv = new_cache(1, 8, 2, 128, 16, x["max_pages"], torch.bfloat16, x["block_table"],
                   num_blocks=x["num_blocks"])
    meta = kv.new_meta()
    bulk_append(kv, x["keys"], x["values"], meta)
    sel, _, _, _ = quest_gpu_step(kv, meta, x, 0, 5, 0.1)
    torch.cuda.synchronize()
    assert sel.cpu().tolist() == [[[0, 1, 2, 3, 4]] * 2]


def test_workspaces_reused_across_steps():
    """The select and attention workspaces keep only arrival counters between
    calls, and every call returns them to zero: reusing one workspace over
    several steps gives the same results as fresh zeroed workspaces."""
    cfg = C5
    x, kv, meta = quest_cache(cfg, 13, 5000, 2)
    x2, kv2, meta2 = quest_cache(cfg, 13, 5000, 2)
    k, scale = 24, W.default_scale(128)
    ws_sel = sp.workspace(sp.SP_OP_SELECT_PAGES, kv, k)
    ws_att = sp.workspace(sp.SP_OP_DECODE_ATTN, kv, k)
    for s in range(3):
        sel_f, _, out_f, lse_f = quest_gpu_step(kv2, meta2, x2, s, k, scale, with_scores=False)
        sp.sp_build_page_meta(kv, x["k_new"][s][:, None].contiguous(),
                              x["v_new"][s][:, None].contiguous(), 1, meta)
        q = x["q"][s].contiguous()
        sel = torch.empty(2, 8, k, dtype=torch.int32, device="cuda")
        sp.sp_select_pages(kv, q, meta, k, sel, None, ws_sel)
        out = torch.empty(2, 64, 128, device="cuda")
        lse = torch.empty(2, 64, device="cuda")
        sp.sp_sparse_decode_attn(kv, q, sel, k, scale, out, lse, ws=ws_att)
        torch.cuda.synchronize()
        assert torch.equal(sel, sel_f)
        assert torch.equal(out, out_f) and torch.equal(lse, lse_f)
    # the counters are back at zero
    nunits = 2 * 8
    assert int(ws_sel[: 4 * nunits].view(torch.int32).abs().sum()) == 0
    assert int(ws_att[: 4 * nunits].view(torch.int32).abs().sum()) == 0


def test_block_table_rows_beyond_lds_staging_match_staged():
    """Block-table rows longer than 8192 pages are not staged in LDS by the
    attention kernel (the block ids are read from global memory instead).
    The same cache seen through a longer table (the extra entries -1) gives
    the same selection and the same attention output bit for bit."""
    x, kv, meta = quest_cache(C2, 17, 1500, 2)
    scale = W.default_scale(128)
    top_k = 24
    sel, scores, out, lse = quest_gpu_step(kv, meta, x, 0, top_k, scale)
    long_bt = torch.full((kv.batch, 8300), -1, dtype=torch.int32, device="cuda")
    long_bt[:, :kv.max_pages] = kv.block_table
    kv_long = sp.PagedKV(kv.k_pool, kv.v_pool, long_bt, kv.seq_lens.clone(), kv.num_q_heads)
    q = x["q"][0].contiguous()
    sel2 = torch.empty_like(sel)
    scores2 = torch.empty(kv.batch, kv.num_kv_heads, kv_long.max_pages, device="cuda")
    sp.sp_select_pages(kv_long, q, meta, top_k, sel2, scores2,
                       sp.workspace(sp.SP_OP_SELECT_PAGES, kv_long, top_k))
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    sp.sp_sparse_decode_attn(kv_long, q, sel, top_k, scale, out2, lse2,
                             ws=sp.workspace(sp.SP_OP_DECODE_ATTN, kv_long, top_k))
    torch.cuda.synchronize()
    assert torch.equal(sel, sel2)
    n_p = scores.shape[2]
    assert torch.equal(scores[:, :, :n_p], scores2[:, :, :n_p])
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
