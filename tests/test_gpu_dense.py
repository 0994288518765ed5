"""GPU parity for dense decode over physically retained slots with ragged
per-sequence lengths (the evicted-state workload), including appends."""
import numpy as np
import pytest
import torch

import kv_cache_selection_sp_amd as sp
import workloads as W
from gpu_util import f64, new_cache, bulk_append
from oracle import dense_decode, attend

pytestmark = pytest.mark.gpu

C4 = W.CONFIGS["evicted_b256_len512to2048"]


def evicted_cache(B, lo, hi, steps, seed, Hq=32, Hkv=8, D=128, dtype=torch.bfloat16):
    cfg = W.EvictedConfig("t", "bf16" if dtype == torch.bfloat16 else "f32", B, Hq, Hkv, D,
                          lo, hi, 8192, steps)
    x = W.evicted_inputs(cfg, seed, device="cuda")
    kv = new_cache(B, Hq, Hkv, D, 16, x["max_pages"], dtype, x["block_table"],
                   num_blocks=x["num_blocks"])
    slot_pos = torch.full((B, Hkv, kv.capacity), -1, dtype=torch.int32, device="cuda")
    bulk_append(kv, x["keys"].to(dtype), x["values"].to(dtype))
    kv.seq_lens.copy_(x["lens"])
    slot_pos[:, :, :hi] = x["positions"]
    return cfg, x, kv, slot_pos


@pytest.mark.parametrize("B,lo,hi", [(5, 1, 70), (3, 200, 600)])
def test_dense_ragged_matches_oracle(B, lo, hi):
    cfg, x, kv, slot_pos = evicted_cache(B, lo, hi, 3, seed=17)
    scale = W.default_scale(128)
    ws = sp.workspace(sp.SP_OP_DECODE_ATTN, kv, 0)
    keys = [[x["keys"][b, h].cpu() for h in range(8)] for b in range(B)]
    vals = [[x["values"][b, h].cpu() for h in range(8)] for b in range(B)]
    lens = x["lens"].cpu().tolist()
    for s in range(cfg.steps):
        pos_new = (x["positions"].max(dim=2).values.max(dim=1).values + 1 + s).to(torch.int32)
        sp.sp_build_page_meta(kv, x["k_new"][s][:, None].contiguous(),
                              x["v_new"][s][:, None].contiguous(), 1, None, pos_new, slot_pos,
                              kv.capacity)
        for b in range(B):
            for h in range(8):
                L = lens[b]
                keys[b][h] = torch.cat([keys[b][h][:L], x["k_new"][s, b, h][None].cpu()])
                vals[b][h] = torch.cat([vals[b][h][:L], x["v_new"][s, b, h][None].cpu()])
            lens[b] += 1
        q = x["q"][s].contiguous()
        out = torch.empty(B, 32, 128, device="cuda")
        lse = torch.empty(B, 32, device="cuda")
        sp.sp_sparse_decode_attn(kv, q, None, 0, scale, out, lse, ws=ws)
        torch.cuda.synchronize()
        assert kv.seq_lens.cpu().tolist() == lens
        ref_out, ref_lse = dense_decode(q.cpu(), keys, vals, lens, scale)
        np.testing.assert_allclose(f64(out), ref_out, atol=2e-3)
        np.testing.assert_allclose(f64(lse), ref_lse, atol=2e-3)


def test_dense_fp32_and_empty_sequence():
    cfg, x, kv, slot_pos = evicted_cache(3, 20, 90, 1, seed=23, Hq=4, Hkv=4, D=64,
                                         dtype=torch.float32)
    kv.seq_lens[1] = 0
    scale = W.default_scale(64)
    ws = sp.workspace(sp.SP_OP_DECODE_ATTN, kv, 0)
    q = x["q"][0].float().contiguous()
    out = torch.empty(3, 4, 64, device="cuda")
    lse = torch.empty(3, 4, device="cuda")
    cap = kv.capacity
    logits = torch.zeros(3, 4, cap, device="cuda")
    sp.sp_sparse_decode_attn(kv, q, None, 0, scale, out, lse, logits, cap, ws)
    torch.cuda.synchronize()
    lens = kv.seq_lens.cpu().tolist()
    keys = [[x["keys"][b, h].float().cpu() for h in range(4)] for b in range(3)]
    vals = [[x["values"][b, h].float().cpu() for h in range(4)] for b in range(3)]
    ref_out, ref_lse = dense_decode(q.cpu(), keys, vals, lens, scale)
    np.testing.assert_allclose(f64(out), ref_out, atol=1e-5)
    assert bool((out[1] == 0).all()) and bool(torch.isneginf(lse[1]).all())
    np.testing.assert_allclose(f64(lse[[0, 2]]), ref_lse[[0, 2]], atol=1e-5)
    for b in (0, 2):
        for a in range(4):
            _, _, _, z = attend(f64(q[b, a]), f64(keys[b][a][:lens[b]]), f64(vals[b][a][:lens[b]]), scale)
            np.testing.assert_allclose(f64(logits[b, a, :lens[b]]), z, atol=1e-5)


@pytest.mark.parametrize("B,lo,hi,Hq,Hkv,dtype", [
    (16, 300, 900, 32, 8, torch.bfloat16),   # units split into a few records (one-pass merge)
    (1, 2500, 3000, 8, 2, torch.bfloat16),   # long units split into many records (batched merge)
    (6, 1, 200, 32, 8, torch.bfloat16),      # short ragged units handled whole
    (3, 20, 300, 8, 8, torch.float32),       # VALU engine
    (2200, 0, 60, 8, 2, torch.bfloat16),     # more sequences than LDS holds: the workspace prefix
])
def test_decode_attn_accumulate_matches_separate_calls(B, lo, hi, Hq, Hkv, dtype):
    """The fused dense attention + H2O score update equals the dense attention
    call followed by the accumulate call, bit for bit: out, lse, logits and
    scores, with the newest slots reset (n_new = 2)."""
    cfg, x, kv, _ = evicted_cache(B, lo, hi, 1, 23, Hq=Hq, Hkv=Hkv, dtype=dtype)
    cap = kv.capacity
    g = torch.Generator(device="cuda").manual_seed(5)
    base = torch.rand(B, Hkv, cap, generator=g, device="cuda")
    q = x["q"][0].to(dtype).contiguous()
    scale = W.default_scale(kv.head_dim)
    ws = sp.workspace(sp.SP_OP_DECODE_ATTN, kv, 0)
    res = []
    for fused in (False, True):
        out = torch.empty(B, Hq, kv.head_dim, device="cuda")
        lse = torch.empty(B, Hq, device="cuda")
        logits = torch.zeros(B, Hq, cap, device="cuda")
        scores = base.clone()
        if fused:
            sp.sp_decode_attn_accumulate(kv, q, scale, out, lse, logits, cap, 2, scores, cap, ws)
        else:
            sp.sp_sparse_decode_attn(kv, q, None, 0, scale, out, lse, logits, cap, ws)
            sp.sp_h2o_accumulate(kv, logits, lse, cap, 2, scores, cap)
        torch.cuda.synchronize()
        res.append((out, lse, logits, scores))
    for a, b in zip(*res):
        assert torch.equal(a, b)
    # the update did happen: slots past a sequence's length keep their old score
    lens = kv.seq_lens.tolist()
    scores = res[1][3]
    for b in range(B):
        assert torch.equal(scores[b, :, lens[b]:], base[b, :, lens[b]:])
        assert bool((scores[b, :, :lens[b]] != base[b, :, :lens[b]]).any()) or lens[b] == 0


def test_dense_batch_beyond_lds_prefix():
    """2500 sequences, more than the attention keeps in LDS (2048): a prefix
    launch writes the tile prefix and each workgroup's first sequence into the
    workspace.  The result equals the same batch attended in two halves
    (prefix in LDS) to 1e-5, and the oracle on sampled sequences, empty ones
    included (zero output, lse = -inf)."""
    B, Hq, Hkv, D = 2500, 8, 2, 128
    cfg = W.EvictedConfig("t", "bf16", B, Hq, Hkv, D, 0, 90, 200, 1)
    x = W.evicted_inputs(cfg, 29, device="cuda")
    kv = new_cache(B, Hq, Hkv, D, 16, x["max_pages"], torch.bfloat16, x["block_table"],
                   num_blocks=x["num_blocks"])
    bulk_append(kv, x["keys"], x["values"])
    kv.seq_lens.copy_(x["lens"])
    q = x["q"][0].contiguous()
    scale = W.default_scale(D)
    out = torch.full((B, Hq, D), float("nan"), device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    print("dense batch 2500", flush=True)
    sp.sp_sparse_decode_attn(kv, q, None, 0, scale, out, lse, ws=sp.workspace(sp.SP_OP_DECODE_ATTN, kv, 0))
    for lo, hi in ((0, 1250), (1250, B)):
        kvh = sp.PagedKV(kv.k_pool, kv.v_pool, kv.block_table[lo:hi].contiguous(), kv.seq_lens[lo:hi].clone(),
                         Hq)
        oh = torch.empty(hi - lo, Hq, D, device="cuda")
        lh = torch.empty(hi - lo, Hq, device="cuda")
        sp.sp_sparse_decode_attn(kvh, q[lo:hi].contiguous(), None, 0, scale, oh, lh,
                                 ws=sp.workspace(sp.SP_OP_DECODE_ATTN, kvh, 0))
        torch.cuda.synchronize()
        torch.testing.assert_close(out[lo:hi], oh, rtol=0, atol=1e-5)
        torch.testing.assert_close(lse[lo:hi], lh, rtol=0, atol=1e-5)
    lens = x["lens"].cpu().tolist()
    empties = [b for b in range(B) if lens[b] == 0]
    assert empties, "the sample has empty sequences"
    G = Hq // Hkv
    for b in [0, 1, 2047, 2048, 2049, B - 1] + empties[:2]:
        for a in range(Hq):
            L = lens[b]
            if L == 0:
                assert bool((out[b, a] == 0).all()) and float(lse[b, a]) == float("-inf")
                continue
            o, l, _, _ = attend(f64(q[b, a]), f64(x["keys"][b, a // G, :L]), f64(x["values"][b, a // G, :L]), scale)
            np.testing.assert_allclose(f64(out[b, a]), o, rtol=0, atol=2e-3)
            assert abs(float(lse[b, a]) - l) <= 2e-3
