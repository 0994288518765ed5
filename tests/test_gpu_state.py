"""GPU: the caller-owned state of a decode loop.

Checkpoint / resume: the whole state lives in the caller's device buffers --
pools, block table, lengths, page summaries, H2O scores and slot positions.
Copied to host memory mid-run and restored into fresh buffers (fresh, zero
workspaces too: the Quest step's epochs start again), the run continues bit
for bit like the uninterrupted one.

Poisoned memory: slots and blocks that no sequence has written, the page
summaries of unused pages, and the split-record area of the attention
workspace, filled with NaN bit patterns, leave every result bit for bit as
with zero-filled memory.  The sequences end inside a page, so the last tile
of each holds unwritten slots (a NaN value times a zero weight would
otherwise reach the output)."""
import pytest
import torch

import kv_cache_selection_sp_amd as sp
import workloads as W
from gpu_util import bulk_append, new_cache

pytestmark = pytest.mark.gpu

NAN = float("nan")


def _snapshot(*tensors):
    torch.cuda.synchronize()
    return [t.cpu() for t in tensors]


def _restore(host):
    # a spare allocation first, so that the restored buffers sit at other addresses
    spare = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    out = [t.to("cuda") for t in host]
    del spare
    return out


# ------------------------------------------------------------------ H2O
def _h2o_setup(fill, B=2, Hq=8, Hkv=2, D=128, P=16, prompt=301, budget=64, window=8, steps=8, seed=7):
    cfg = W.H2OConfig("t", "bf16", B, Hq, Hkv, D, prompt, budget, window, steps, page_size=P)
    x = W.h2o_inputs(cfg, seed, device="cuda")
    kv = new_cache(B, Hq, Hkv, D, P, x["max_pages"], torch.bfloat16, x["block_table"],
                   num_blocks=x["num_blocks"])
    kv.k_pool.fill_(fill)
    kv.v_pool.fill_(fill)
    cap = kv.capacity
    scores = torch.full((B, Hkv, cap), fill, device="cuda")
    slot_pos = torch.full((B, Hkv, cap), -1, dtype=torch.int32, device="cuda")
    scale = W.default_scale(D)
    bulk_append(kv, x["keys"], x["values"], None, None, slot_pos, cap)
    scores[:, :, :prompt] = 0.0
    sp.sp_h2o_prefill_scores(kv, x["q_prompt"], prompt, scale, scores, cap,
                             sp.workspace(sp.SP_OP_H2O_PREFILL, kv, prompt))
    sp.sp_h2o_evict_compact(kv, scores, slot_pos, cap, budget, window, sp.workspace(sp.SP_OP_H2O_EVICT, kv, budget))
    return cfg, x, kv, scores, slot_pos, scale


def _h2o_steps(cfg, x, kv, scores, slot_pos, scale, s0, s1, poison_ws=False):
    B, Hq, D, cap = kv.batch, kv.num_q_heads, kv.head_dim, kv.capacity
    ws_a = sp.workspace(sp.SP_OP_DECODE_ATTN, kv, 0)
    if poison_ws:
        # the split records behind the per-unit counters (which must start at zero)
        cb = (B * kv.num_kv_heads * 4 + 255) // 256 * 256
        ws_a.view(torch.uint8)[cb:].view(torch.float32).fill_(NAN)
    ws_e = sp.workspace(sp.SP_OP_H2O_EVICT, kv, cfg.budget)
    res = []
    for s in range(s0, s1):
        pos_new = torch.full((B,), cfg.prompt + s, dtype=torch.int32, device="cuda")
        sp.sp_build_page_meta(kv, x["k_new"][s][:, None].contiguous(), x["v_new"][s][:, None].contiguous(), 1,
                              None, pos_new, slot_pos, cap)
        out = torch.empty(B, Hq, D, device="cuda")
        lse = torch.empty(B, Hq, device="cuda")
        logits = torch.zeros(B, Hq, cap, device="cuda")
        sp.sp_decode_attn_accumulate(kv, x["q"][s].contiguous(), scale, out, lse, logits, cap, 1, scores, cap, ws_a)
        L = int(kv.seq_lens[0])
        res.append((out, lse, logits[:, :, :L].clone(), scores[:, :, :L].clone()))
        sp.sp_h2o_evict_compact(kv, scores, slot_pos, cap, cfg.budget, cfg.recent_window, ws_e)
    torch.cuda.synchronize()
    return res


def _live_h2o(kv, scores, slot_pos):
    """The valid part of the H2O state: per (sequence, KV head) its first
    seq_len slots' positions, scores, keys and values."""
    torch.cuda.synchronize()
    out = []
    for b in range(kv.batch):
        L = int(kv.seq_lens[b])
        for h in range(kv.num_kv_heads):
            k_, v_ = sp.read_slots(kv, b, h, L)
            out += [slot_pos[b, h, :L].cpu(), scores[b, h, :L].cpu(), k_.cpu(), v_.cpu()]
    return out


def _equal_lists(a, b):
    assert len(a) == len(b)
    for x_, y_ in zip(a, b):
        for p, q in zip(x_ if isinstance(x_, (tuple, list)) else (x_,), y_ if isinstance(y_, (tuple, list)) else (y_,)):
            assert torch.equal(p, q)


def test_h2o_checkpoint_resume_is_bit_exact():
    cfg, x, kv, scores, slot_pos, scale = _h2o_setup(0.0)
    _h2o_steps(cfg, x, kv, scores, slot_pos, scale, 0, 3)
    host = _snapshot(kv.k_pool, kv.v_pool, kv.block_table, kv.seq_lens, scores, slot_pos)
    ref = _h2o_steps(cfg, x, kv, scores, slot_pos, scale, 3, 6)
    ref_state = _live_h2o(kv, scores, slot_pos)
    k2, v2, bt2, lens2, scores2, slot2 = _restore(host)
    kv2 = sp.PagedKV(k2, v2, bt2, lens2, kv.num_q_heads)
    got = _h2o_steps(cfg, x, kv2, scores2, slot2, scale, 3, 6)
    _equal_lists(ref, got)
    _equal_lists(ref_state, _live_h2o(kv2, scores2, slot2))


def test_h2o_poisoned_memory_leaves_results_unchanged():
    """A 57-token prompt under a 64-slot budget: the first steps attend over
    a last tile with unwritten slots, the later ones evict."""
    runs = []
    for fill, poison_ws in ((0.0, False), (NAN, True)):
        cfg, x, kv, scores, slot_pos, scale = _h2o_setup(fill, prompt=57, steps=10)
        res = _h2o_steps(cfg, x, kv, scores, slot_pos, scale, 0, 10, poison_ws=poison_ws)
        runs.append((res, _live_h2o(kv, scores, slot_pos)))
    for (o, l, lg, sc) in runs[1][0]:
        assert torch.isfinite(o).all() and torch.isfinite(l).all()
    _equal_lists(runs[0][0], runs[1][0])
    _equal_lists(runs[0][1], runs[1][1])


# ------------------------------------------------------------------ Quest
C2 = W.CONFIGS["quest_llama3_8b_b16_ctx32k"]
C5 = W.CONFIGS["quest_gqa8_b4_ctx128k"]


def _quest_setup(cfg, context, batch, fill, seed=11):
    x = W.quest_inputs(cfg, seed, device="cuda", context=context, batch=batch)
    kv = new_cache(batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size, x["max_pages"],
                   W.torch_dtype(cfg.dtype), x["block_table"], num_blocks=x["num_blocks"])
    kv.k_pool.fill_(fill)
    kv.v_pool.fill_(fill)
    meta = kv.new_meta()
    meta.fill_(fill)
    bulk_append(kv, x["keys"], x["values"], meta)
    return x, kv, meta


def _quest_steps(cfg, x, kv, meta, s0, s1, top_k, single=True, poison_ws=False, n_recent=0):
    B, Hq, H, D = kv.batch, kv.num_q_heads, kv.num_kv_heads, kv.head_dim
    scale = W.default_scale(D)
    res = []
    if single:
        ws = sp.workspace(sp.SP_OP_QUEST_STEP, kv, top_k)
    else:
        ws_s = sp.workspace(sp.SP_OP_SELECT_PAGES, kv, top_k)
        ws_a = sp.workspace(sp.SP_OP_DECODE_ATTN, kv, top_k)
        if poison_ws:
            cb = (B * H * 4 + 255) // 256 * 256
            ws_a.view(torch.uint8)[cb:].view(torch.float32).fill_(NAN)
    for s in range(s0, s1):
        kn, vn, q = x["k_new"][s].contiguous(), x["v_new"][s].contiguous(), x["q"][s].contiguous()
        sel = torch.empty(B, H, top_k, dtype=torch.int32, device="cuda")
        sc = torch.empty(B, H, kv.max_pages, device="cuda")
        out = torch.empty(B, Hq, D, device="cuda")
        lse = torch.empty(B, Hq, device="cuda")
        if single:
            sp.sp_quest_decode_step(kv, kn, vn, None, None, 0, meta, q, top_k, 0, n_recent, sp.SP_GROUP_SUM, scale,
                                    sel, sc, out, lse, ws)
        else:
            sp.sp_append_select_pages(kv, kn, vn, None, None, 0, meta, q, top_k, 0, n_recent, sp.SP_GROUP_SUM, sel,
                                      sc, ws_s)
            sp.sp_sparse_decode_attn(kv, q, sel, top_k, scale, out, lse, ws=ws_a)
        L = int(kv.seq_lens.max())
        res.append((sel, sc[:, :, :(L + kv.page_size - 1) // kv.page_size].clone(), out, lse))
    torch.cuda.synchronize()
    if single:
        assert sp.sp_quest_step_error(kv, ws) == 0
    return res


@pytest.mark.parametrize("cfg,context,batch,top_k", [(C2, 1999, 3, 16), (C5, 2999, 2, 24)])
def test_quest_step_checkpoint_resume_is_bit_exact(cfg, context, batch, top_k):
    x, kv, meta = _quest_setup(cfg, context, batch, 0.0)
    _quest_steps(cfg, x, kv, meta, 0, 2, top_k)
    host = _snapshot(kv.k_pool, kv.v_pool, kv.block_table, kv.seq_lens, meta)
    ref = _quest_steps(cfg, x, kv, meta, 2, 4, top_k)
    k2, v2, bt2, lens2, meta2 = _restore(host)
    kv2 = sp.PagedKV(k2, v2, bt2, lens2, kv.num_q_heads)
    assert sp.sp_quest_step_single_launch(kv2)
    got = _quest_steps(cfg, x, kv2, meta2, 2, 4, top_k)
    _equal_lists(ref, got)


@pytest.mark.parametrize("single", [True, False])
@pytest.mark.parametrize("cfg,context,batch,top_k", [(C2, 2000, 3, 16), (C5, 3000, 2, 24), (C2, 100, 2, 16)])
def test_quest_poisoned_memory_leaves_results_unchanged(cfg, context, batch, top_k, single):
    """The newest page is always selected (one forced recent page), and it
    ends inside the page on every step."""
    runs = []
    for fill, poison_ws in ((0.0, False), (NAN, True)):
        x, kv, meta = _quest_setup(cfg, context, batch, fill)
        runs.append(_quest_steps(cfg, x, kv, meta, 0, 3, top_k, single=single, poison_ws=poison_ws, n_recent=1))
    for (sel, sc, out, lse) in runs[1]:
        assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    _equal_lists(runs[0], runs[1])


def test_masked_attention_poisoned_memory_leaves_results_unchanged():
    """OmniKV's sparse layer: token masks with holes over pools whose
    unwritten slots hold NaN bit patterns."""
    B, Hq, H, D, P, n = 2, 8, 2, 128, 16, 501
    outs = []
    for fill in (0.0, NAN):
        g = torch.Generator(device="cuda")
        g.manual_seed(3)
        keys = torch.randn(B, H, n, D, generator=g, device="cuda").to(torch.bfloat16)
        values = torch.randn(B, H, n, D, generator=g, device="cuda").to(torch.bfloat16)
        q = torch.randn(B, Hq, D, generator=g, device="cuda").to(torch.bfloat16)
        max_pages = -(-n // P)
        bt, nblk = W.random_block_table(B, max_pages + 3, g, "cuda")
        kv = new_cache(B, Hq, H, D, P, max_pages + 3, torch.bfloat16, bt, num_blocks=nblk)
        kv.k_pool.fill_(fill)
        kv.v_pool.fill_(fill)
        bulk_append(kv, keys, values)
        # every page, with a mask of alternate tokens (the last page's mask
        # reaches past the sequence's end only through its valid tokens)
        k_pages = max_pages
        pages = torch.arange(k_pages, dtype=torch.int32, device="cuda").repeat(B, H, 1).contiguous()
        mask = torch.full((B, H, k_pages), 0x5555, dtype=torch.int32, device="cuda")
        last = n - (k_pages - 1) * P
        mask[:, :, -1] &= (1 << last) - 1
        out = torch.empty(B, Hq, D, device="cuda")
        lse = torch.empty(B, Hq, device="cuda")
        sp.sp_sparse_decode_attn_masked(kv, q, pages, mask, k_pages, W.default_scale(D), out, lse,
                                        sp.workspace(sp.SP_OP_DECODE_ATTN, kv, k_pages))
        torch.cuda.synchronize()
        outs.append((out, lse))
    assert torch.isfinite(outs[1][0]).all()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
