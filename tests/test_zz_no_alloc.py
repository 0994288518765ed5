"""The allocation-free attention, sp_sparse_decode_attn_noalloc, through the C
ABI: its counters and split records live in the library's per-device scratch
array instead of a caller workspace, with the same kernels, so every output
equals sp_sparse_decode_attn's bit for bit.  Two calls in a row per mode, the
second on a smaller cache (the array keeps the first call's records; its
counters must be back at zero)."""
import pytest
import torch

import kv_cache_selection_sp_amd as sp
import workloads as W
from gpu_util import bulk_append, new_cache, quest_cache

pytestmark = pytest.mark.gpu

QUEST = W.CONFIGS["quest_llama3_8b_b16_ctx32k"]


def _quest_pair(seed, context, batch, top_k):
    x, kv, meta = quest_cache(QUEST, seed, context=context, batch=batch)
    sel = torch.empty(batch, kv.num_kv_heads, top_k, dtype=torch.int32, device="cuda")
    q = x["q"][0].contiguous()
    sp.sp_select_pages(kv, q, meta, top_k, sel, None, sp.workspace(sp.SP_OP_SELECT_PAGES, kv, top_k))
    scale = W.default_scale(kv.head_dim)
    res = []
    for noalloc in (False, True):
        out = torch.full((batch, kv.num_q_heads, kv.head_dim), float("nan"), device="cuda")
        lse = torch.full((batch, kv.num_q_heads), float("nan"), device="cuda")
        if noalloc:
            sp.sp_sparse_decode_attn_noalloc(kv, q, sel, top_k, scale, out, lse)
        else:
            sp.sp_sparse_decode_attn(kv, q, sel, top_k, scale, out, lse,
                                     ws=sp.workspace(sp.SP_OP_DECODE_ATTN, kv, top_k))
        torch.cuda.synchronize()
        res.append((out, lse))
    return res


def test_noalloc_sparse_two_calls_second_smaller():
    print("noalloc sparse: B=4 ctx 6000 k=128, then B=2 ctx 3000 k=64", flush=True)
    for seed, context, batch, top_k in ((31, 6000, 4, 128), (32, 3000, 2, 64)):
        (o_ws, l_ws), (o_na, l_na) = _quest_pair(seed, context, batch, top_k)
        assert torch.isfinite(o_ws).all() and torch.isfinite(l_ws).all()
        assert torch.equal(o_ws, o_na) and torch.equal(l_ws, l_na)


def _dense_pair(seed, B, lo, hi):
    cfg = W.EvictedConfig("t", "bf16", B, 32, 8, 128, lo, hi, 8192, 1)
    x = W.evicted_inputs(cfg, seed, device="cuda")
    kv = new_cache(B, 32, 8, 128, 16, x["max_pages"], torch.bfloat16, x["block_table"],
                   num_blocks=x["num_blocks"])
    bulk_append(kv, x["keys"].to(torch.bfloat16), x["values"].to(torch.bfloat16))
    kv.seq_lens.copy_(x["lens"])
    q = x["q"][0].contiguous()
    cap = kv.capacity
    scale = W.default_scale(128)
    res = []
    for noalloc in (False, True):
        out = torch.full((B, 32, 128), float("nan"), device="cuda")
        lse = torch.full((B, 32), float("nan"), device="cuda")
        logits = torch.zeros(B, 32, cap, device="cuda")
        if noalloc:
            sp.sp_sparse_decode_attn_noalloc(kv, q, None, 0, scale, out, lse, logits, cap)
        else:
            sp.sp_sparse_decode_attn(kv, q, None, 0, scale, out, lse, logits, cap,
                                     sp.workspace(sp.SP_OP_DECODE_ATTN, kv, 0))
        torch.cuda.synchronize()
        res.append((out, lse, logits))
    return res


def test_noalloc_dense_with_logits_two_calls_second_smaller():
    print("noalloc dense: B=12 lens 300..1500 with logits, then B=3 lens 20..400", flush=True)
    for seed, B, lo, hi in ((41, 12, 300, 1500), (42, 3, 20, 400)):
        ws_res, na_res = _dense_pair(seed, B, lo, hi)
        assert torch.isfinite(ws_res[0]).all()
        for a, b in zip(ws_res, na_res):
            assert torch.equal(a, b)
