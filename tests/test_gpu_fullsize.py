"""GPU parity at the full workload sizes, in the launch configuration that
bench.py times (the kernels pick their workgroup shape and split from the
sizes), checked on sampled (sequence, KV head) units that the oracle computes
one by one."""
import numpy as np
import pytest
import torch

import kv_cache_selection_sp_amd as sp
import workloads as W
from gpu_util import TOL, f64, check_selection
from oracle import attend, quest_decode_head, h2o_retain

pytestmark = pytest.mark.gpu


def _quest_full(name, samples):
    cfg = W.CONFIGS[name]
    x = W.quest_inputs(cfg, W.config_seed(name), device="cuda")
    B, H, Hq, D, P, k = x["batch"], cfg.num_kv_heads, cfg.num_q_heads, cfg.head_dim, cfg.page_size, cfg.top_k
    G = Hq // H
    dt = W.torch_dtype(cfg.dtype)
    kv = sp.PagedKV.allocate(B, Hq, H, D, P, x["max_pages"], x["num_blocks"], dt, x["block_table"])
    meta = kv.new_meta()
    sp.sp_build_page_meta(kv, x["keys"].permute(0, 2, 1, 3).contiguous(),
                          x["values"].permute(0, 2, 1, 3).contiguous(), x["context"], meta)
    sp.sp_build_page_meta(kv, x["k_new"][0][:, None].contiguous(), x["v_new"][0][:, None].contiguous(),
                          1, meta)
    q = x["q"][0].contiguous()
    sel = torch.empty(B, H, k, dtype=torch.int32, device="cuda")
    scores = torch.empty(B, H, kv.max_pages, device="cuda")
    sp.sp_select_pages(kv, q, meta, k, sel, scores, sp.workspace(sp.SP_OP_SELECT_PAGES, kv, k))
    out = torch.empty(B, Hq, D, device="cuda")
    lse = torch.empty(B, Hq, device="cuda")
    scale = W.default_scale(D)
    sp.sp_sparse_decode_attn(kv, q, sel, k, scale, out, lse, ws=sp.workspace(sp.SP_OP_DECODE_ATTN, kv, k))
    torch.cuda.synchronize()
    L = x["context"] + 1
    for (b, h) in samples:
        keys = torch.cat([x["keys"][b, h], x["k_new"][0, b, h][None]]).cpu()
        vals = torch.cat([x["values"][b, h], x["v_new"][0, b, h][None]]).cpu()
        qs = f64(q[b, h * G:(h + 1) * G])
        r = quest_decode_head(qs, keys, vals, P, k, scale)
        check_selection(sel[b, h].cpu(), r["scores"], k)
        pages = [int(p) for p in sel[b, h].cpu() if p >= 0]
        toks = np.concatenate([np.arange(p * P, min(L, (p + 1) * P)) for p in pages])
        kk, vv = f64(keys)[toks], f64(vals)[toks]
        for a in range(G):
            o, l, _, _ = attend(qs[a], kk, vv, scale)
            np.testing.assert_allclose(f64(out[b, h * G + a]), o, rtol=0, atol=TOL[dt])
            assert abs(float(lse[b, h * G + a]) - l) <= TOL[dt]


def test_quest_llama3_8b_full_size_sampled_units():
    _quest_full("quest_llama3_8b_b16_ctx32k", [(0, 0), (3, 5), (7, 7), (11, 2), (15, 3)])


def test_quest_gqa8_full_size_sampled_units():
    _quest_full("quest_gqa8_b4_ctx128k", [(0, 0), (1, 6), (3, 7)])


def test_h2o_full_size_prompt_compaction_and_step():
    name = "h2o_qwen3_8b_b32_prompt8k_bud1k"
    cfg = W.CONFIGS[name]
    x = W.h2o_inputs(cfg, W.config_seed(name), device="cuda", steps=1)
    B, H, Hq, D, G = x["batch"], cfg.num_kv_heads, cfg.num_q_heads, cfg.head_dim, cfg.group
    n, bud, win = x["prompt"], cfg.budget, cfg.recent_window
    kv = sp.PagedKV.allocate(B, Hq, H, D, 16, x["max_pages"], x["num_blocks"], torch.bfloat16,
                             x["block_table"])
    cap = kv.capacity
    scores = torch.zeros(B, H, cap, device="cuda")
    slot_pos = torch.zeros(B, H, cap, dtype=torch.int32, device="cuda")
    sp.sp_build_page_meta(kv, x["keys"].permute(0, 2, 1, 3).contiguous(),
                          x["values"].permute(0, 2, 1, 3).contiguous(), n, None, None, slot_pos, cap)
    scores[:, :, :n] = x["prompt_scores"]
    sp.sp_h2o_evict_compact(kv, scores, slot_pos, cap, bud, win)
    pos_new = torch.full((B,), n, dtype=torch.int32, device="cuda")
    sp.sp_build_page_meta(kv, x["k_new"][0][:, None].contiguous(), x["v_new"][0][:, None].contiguous(),
                          1, None, pos_new, slot_pos, cap)
    q = x["q"][0].contiguous()
    out = torch.empty(B, Hq, D, device="cuda")
    lse = torch.empty(B, Hq, device="cuda")
    logits = torch.empty(B, Hq, cap, device="cuda")
    scale = W.default_scale(D)
    sp.sp_sparse_decode_attn(kv, q, None, 0, scale, out, lse, logits, cap,
                             sp.workspace(sp.SP_OP_DECODE_ATTN, kv, 0))
    torch.cuda.synchronize()
    assert bool((kv.seq_lens == bud + 1).all())
    ps = x["prompt_scores"].cpu().double().numpy()
    for (b, h) in [(0, 0), (9, 4), (31, 7)]:
        # fp32 scores on both sides and ties by lower slot (= position here): exact
        keep = h2o_retain(np.arange(n), ps[b, h].astype(np.float32).astype(np.float64), bud, win)
        pos = slot_pos[b, h, :bud].cpu().numpy()
        assert pos.tolist() == keep
        keys = torch.cat([x["keys"][b, h].cpu()[keep], x["k_new"][0, b, h][None].cpu()])
        vals = torch.cat([x["values"][b, h].cpu()[keep], x["v_new"][0, b, h][None].cpu()])
        for a in range(h * G, (h + 1) * G):
            o, l, _, z = attend(f64(q[b, a]), f64(keys), f64(vals), scale)
            np.testing.assert_allclose(f64(out[b, a]), o, rtol=0, atol=2e-3)
            assert abs(float(lse[b, a]) - l) <= 2e-3
            np.testing.assert_allclose(f64(logits[b, a, :bud + 1]), z, rtol=0, atol=1e-4)


def test_evicted_full_size_sampled_sequences():
    name = "evicted_b256_len512to2048"
    cfg = W.CONFIGS[name]
    x = W.evicted_inputs(cfg, W.config_seed(name), device="cuda", steps=1)
    B, H, Hq, D, G = x["batch"], cfg.num_kv_heads, cfg.num_q_heads, cfg.head_dim, cfg.group
    kv = sp.PagedKV.allocate(B, Hq, H, D, 16, x["max_pages"], x["num_blocks"], torch.bfloat16,
                             x["block_table"])
    sp.sp_build_page_meta(kv, x["keys"].permute(0, 2, 1, 3).contiguous(),
                          x["values"].permute(0, 2, 1, 3).contiguous(), cfg.max_len, None)
    kv.seq_lens.copy_(x["lens"])
    q = x["q"][0].contiguous()
    out = torch.empty(B, Hq, D, device="cuda")
    lse = torch.empty(B, Hq, device="cuda")
    scale = W.default_scale(D)
    sp.sp_sparse_decode_attn(kv, q, None, 0, scale, out, lse, ws=sp.workspace(sp.SP_OP_DECODE_ATTN, kv, 0))
    torch.cuda.synchronize()
    lens = x["lens"].cpu().tolist()
    for b in (0, 77, 128, 255):
        L = lens[b]
        for h in (0, 7):
            kk, vv = f64(x["keys"][b, h, :L]), f64(x["values"][b, h, :L])
            for a in range(h * G, (h + 1) * G):
                o, l, _, _ = attend(f64(q[b, a]), kk, vv, scale)
                np.testing.assert_allclose(f64(out[b, a]), o, rtol=0, atol=2e-3)
                assert abs(float(lse[b, a]) - l) <= 2e-3
