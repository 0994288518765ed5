"""HIP-graph replay of whole decode steps: every call of the library is
stream-ordered and capturable (no host synchronisation, no allocation, no
memset), so a step captured once and replayed with fresh inputs in
address-stable buffers must give bit-identical results to eager launches.
Each replay is checked, with eager work and synchronisations in between."""
import pytest
import torch

import kv_cache_selection_sp_amd as sp
import workloads as W
from gpu_util import quest_cache, new_cache, bulk_append

pytestmark = pytest.mark.gpu

C2 = W.CONFIGS["quest_llama3_8b_b16_ctx32k"]
C3 = W.CONFIGS["h2o_qwen3_8b_b32_prompt8k_bud1k"]


@pytest.mark.parametrize("form", ["three_calls", "single_launch"])
def test_quest_step_graph_replay_matches_eager(form):
    """single_launch: the step as the bench runs it (sp_quest_decode_step);
    three_calls: append, select, attend."""
    B, k, steps = 2, 16, 4
    scale = W.default_scale(128)
    xa, kva, meta_a = quest_cache(C2, 77, 3000, B)
    xb, kvb, meta_b = quest_cache(C2, 77, 3000, B)
    bufs = {}
    for name, kv in (("a", kva), ("b", kvb)):
        bufs[name] = dict(
            q=torch.empty(B, 32, 128, dtype=torch.bfloat16, device="cuda"),
            kn=torch.empty(B, 1, 8, 128, dtype=torch.bfloat16, device="cuda"),
            vn=torch.empty(B, 1, 8, 128, dtype=torch.bfloat16, device="cuda"),
            sel=torch.empty(B, 8, k, dtype=torch.int32, device="cuda"),
            out=torch.empty(B, 32, 128, device="cuda"),
            lse=torch.empty(B, 32, device="cuda"),
            ws_sel=sp.workspace(sp.SP_OP_SELECT_PAGES, kv, k),
            ws_att=sp.workspace(sp.SP_OP_DECODE_ATTN, kv, k),
            ws_step=sp.workspace(sp.SP_OP_QUEST_STEP, kv, k))

    def step(kv, meta, t):
        if form == "single_launch":
            sp.sp_quest_decode_step(kv, t["kn"][:, 0], t["vn"][:, 0], None, None, 0, meta, t["q"], k, 0, 0,
                                    sp.SP_GROUP_SUM, scale, t["sel"], None, t["out"], t["lse"], t["ws_step"])
            return
        sp.sp_build_page_meta(kv, t["kn"], t["vn"], 1, meta)
        sp.sp_select_pages(kv, t["q"], meta, k, t["sel"], None, t["ws_sel"])
        sp.sp_sparse_decode_attn(kv, t["q"], t["sel"], k, scale, t["out"], t["lse"], ws=t["ws_att"])

    def load(t, x, s):
        t["q"].copy_(x["q"][s])
        t["kn"].copy_(x["k_new"][s][:, None])
        t["vn"].copy_(x["v_new"][s][:, None])

    g = torch.cuda.CUDAGraph()
    load(bufs["b"], xb, 0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step(kvb, meta_b, bufs["b"])
    for s in range(steps):
        load(bufs["a"], xa, s)
        step(kva, meta_a, bufs["a"])
        load(bufs["b"], xb, s)
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()       # eager work between replays
        torch.cuda.synchronize()
        del junk
        for key in ("sel", "out", "lse"):
            assert torch.equal(bufs["a"][key], bufs["b"][key]), (s, key)
        assert torch.equal(kva.seq_lens, kvb.seq_lens)
        assert torch.equal(meta_a, meta_b)


@pytest.mark.parametrize("fused", [False, True])
def test_h2o_step_graph_replay_matches_eager(fused):
    """fused: the step as the bench runs it -- attention and score update in
    one launch (sp_decode_attn_accumulate), the eviction's length update in
    its kernel (per-sequence counters in its workspace)."""
    B, Hq, Hkv, D, prompt, budget, window = 2, 8, 2, 128, 300, 64, 8
    cfg = W.H2OConfig("t", "bf16", B, Hq, Hkv, D, prompt, budget, window, 4)
    x = W.h2o_inputs(cfg, 5, device="cuda")
    scale = W.default_scale(D)
    state = {}
    for name in ("a", "b"):
        kv = new_cache(B, Hq, Hkv, D, 16, x["max_pages"], torch.bfloat16, x["block_table"],
                       num_blocks=x["num_blocks"])
        cap = kv.capacity
        slot_pos = torch.zeros(B, Hkv, cap, dtype=torch.int32, device="cuda")
        scores = torch.zeros(B, Hkv, cap, device="cuda")
        bulk_append(kv, x["keys"], x["values"], None, None, slot_pos, cap)
        # prefill scores of the prompt (one causal chunk), then the compaction
        sp.sp_h2o_prefill_scores(kv, x["q_prompt"], prompt, scale, scores, cap,
                                 sp.workspace(sp.SP_OP_H2O_PREFILL, kv, prompt))
        sp.sp_h2o_evict_compact(kv, scores, slot_pos, cap, budget, window)
        state[name] = dict(kv=kv, cap=cap, slot_pos=slot_pos, scores=scores,
                           q=torch.empty(B, Hq, D, dtype=torch.bfloat16, device="cuda"),
                           kn=torch.empty(B, 1, Hkv, D, dtype=torch.bfloat16, device="cuda"),
                           vn=torch.empty(B, 1, Hkv, D, dtype=torch.bfloat16, device="cuda"),
                           pos=torch.zeros(B, dtype=torch.int32, device="cuda"),
                           out=torch.empty(B, Hq, D, device="cuda"),
                           lse=torch.empty(B, Hq, device="cuda"),
                           logits=torch.zeros(B, Hq, cap, device="cuda"),
                           ws=sp.workspace(sp.SP_OP_DECODE_ATTN, kv, 0),
                           ws_e=sp.workspace(sp.SP_OP_H2O_EVICT, kv, budget) if fused else None)

    def step(t):
        kv, cap = t["kv"], t["cap"]
        sp.sp_build_page_meta(kv, t["kn"], t["vn"], 1, None, t["pos"], t["slot_pos"], cap)
        if fused:
            sp.sp_decode_attn_accumulate(kv, t["q"], scale, t["out"], t["lse"], t["logits"], cap, 1,
                                         t["scores"], cap, t["ws"])
        else:
            sp.sp_sparse_decode_attn(kv, t["q"], None, 0, scale, t["out"], t["lse"], t["logits"], cap, t["ws"])
            sp.sp_h2o_accumulate(kv, t["logits"], t["lse"], cap, 1, t["scores"], cap)
        sp.sp_h2o_evict_compact(kv, t["scores"], t["slot_pos"], cap, budget, window, t["ws_e"])

    def load(t, s):
        t["q"].copy_(x["q"][s])
        t["kn"].copy_(x["k_new"][s][:, None])
        t["vn"].copy_(x["v_new"][s][:, None])
        t["pos"].fill_(prompt + s)

    g = torch.cuda.CUDAGraph()
    load(state["b"], 0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step(state["b"])
    for s in range(4):
        load(state["a"], s)
        step(state["a"])
        load(state["b"], s)
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        del junk
        a, b = state["a"], state["b"]
        for key in ("out", "lse", "slot_pos", "scores"):
            assert torch.equal(a[key], b[key]), (s, key)
        assert torch.equal(a["kv"].seq_lens, b["kv"].seq_lens)
        assert torch.equal(a["kv"].k_pool, b["kv"].k_pool) and torch.equal(a["kv"].v_pool, b["kv"].v_pool)
