"""GPU parity of SnapKV prompt selection: window scores and pooling
(sp_snapkv_scores) against the fp64 oracle, the retained set after
compaction (sp_h2o_evict_compact with the window as the protected recent
window) against the oracle's retention rule, and decoding over the result.

Score tolerance: 1e-5 relative (plus 1e-7 absolute for tiny values).  The
largest error observed over these cases is 1.4e-6 relative (each logit is an
fp32 sum of D exact bf16 products, and the normalisers and probabilities are
fp32).  Retained sets: equal to the oracle's except candidates within
1e-5 * max(|cutoff|, 1) of the cutoff pooled score; none has differed (max
pooling copies one u value to up to kappa neighbours, so exact ties are
common; both sides break them by position).  The BAND lines printed under -s
record the observed errors and band counts.
"""
import dataclasses

import numpy as np
import pytest
import torch

import kv_cache_selection_sp_amd as sp
import workloads as W
from gpu_util import f64
from oracle import attend, snapkv_pool, snapkv_retain, snapkv_window_scores

pytestmark = pytest.mark.gpu

SMALL = W.CONFIGS["snapkv_b2_h8_kv2_d128_prompt2k"]
RTOL, ATOL = 1e-5, 1e-7
SENTINEL = -7.0


def _cache(cfg, x, lens=None):
    B, H, Hq, D, P = x["batch"], cfg.num_kv_heads, cfg.num_q_heads, cfg.head_dim, cfg.page_size
    kv = sp.PagedKV.allocate(B, Hq, H, D, P, x["max_pages"], x["num_blocks"], torch.bfloat16,
                             x["block_table"])
    cap = kv.capacity
    slot_pos = torch.zeros(B, H, cap, dtype=torch.int32, device="cuda")
    n = x["prompt"]
    sp.sp_build_page_meta(kv, x["keys"].permute(0, 2, 1, 3).contiguous(),
                          x["values"].permute(0, 2, 1, 3).contiguous(), n, None, None, slot_pos, cap)
    if lens is not None:
        kv.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
    return kv, slot_pos


def _scores(cfg, kv, x, w=None, kappa=None, n_sink=None):
    w = cfg.window if w is None else w
    kappa = cfg.pool_kernel if kappa is None else kappa
    n_sink = cfg.n_sink if n_sink is None else n_sink
    cap = kv.capacity
    scores = torch.full((kv.batch, kv.num_kv_heads, cap), SENTINEL, device="cuda")
    q_obs = x["q_obs"][:, :w].contiguous()
    sp.sp_snapkv_scores(kv, q_obs, w, W.default_scale(cfg.head_dim), kappa, n_sink, scores, cap,
                        sp.workspace(sp.SP_OP_SNAPKV_SCORES, kv, w))
    torch.cuda.synchronize()
    return scores


def _oracle_pooled(cfg, x, b, h, L, w, kappa, n_sink):
    G = cfg.group
    q = f64(x["q_obs"][b, :w, h * G:(h + 1) * G])
    keys = f64(x["keys"][b, h, :L])
    u = snapkv_window_scores(q, keys, W.default_scale(cfg.head_dim))
    s = snapkv_pool(u, kappa)
    s[:min(n_sink, len(s))] = np.inf
    return u, s


def _check_scores(got_row, ref, L, w):
    got = f64(got_row)
    Le = max(L - w, 0)
    if Le:
        fin = np.isfinite(ref)
        assert np.array_equal(np.isinf(got[:Le]), ~fin)
        err = np.abs(got[:Le][fin] - ref[fin])
        if fin.any():
            print(f"BAND snapkv score max_rel {float((err / np.maximum(np.abs(ref[fin]), 1e-30)).max()):.3e} "
                  f"max_abs {float(err.max()):.3e}")
        assert bool((err <= RTOL * np.abs(ref[fin]) + ATOL).all()), float((err / np.abs(ref[fin])).max())
    assert bool((got[Le:] == SENTINEL).all())          # window and beyond: not written


def _check_retained(pos, pooled, n, budget, w, n_sink):
    """pos: the GPU's slot positions of slots [0, budget) after compaction."""
    keep_ref = snapkv_retain(n, pooled, budget, w, n_sink)
    got = [int(p) for p in pos]
    assert got == sorted(got) and len(set(got)) == len(got) == min(n, budget)
    if n <= budget:
        assert got == keep_ref
        return
    Le = n - w
    assert set(range(Le, n)) <= set(got)
    assert set(range(min(n_sink, Le))) <= set(got)
    diff = set(got) ^ set(keep_ref)
    rest = np.sort(pooled[n_sink:Le])[::-1]
    if budget - w - min(n_sink, Le) >= 1:
        cut = rest[budget - w - min(n_sink, Le) - 1]
        inband = int(np.sum(np.abs(pooled[n_sink:Le] - cut) <= 1e-5 * max(abs(cut), 1.0)))
        print(f"BAND snapkv retain in_1e-5_band {inband} diff {len(diff)}")
    if diff:
        cutoff = rest[budget - w - min(n_sink, Le) - 1]
        for j in diff:
            assert abs(pooled[j] - cutoff) <= 1e-5 * max(abs(cutoff), 1.0), (j, pooled[j], cutoff)


def test_snapkv_scores_small_ragged():
    cfg = SMALL
    x = W.snapkv_inputs(cfg, W.config_seed(cfg.name), device="cuda", steps=1)
    lens = [2048, 1543]
    kv, _ = _cache(cfg, x, lens)
    scores = _scores(cfg, kv, x)
    for b in range(2):
        for h in range(cfg.num_kv_heads):
            _, s = _oracle_pooled(cfg, x, b, h, lens[b], cfg.window, cfg.pool_kernel, 0)
            _check_scores(scores[b, h], s, lens[b], cfg.window)


@pytest.mark.parametrize("Hq,Hkv,D,P,w,kappa,n_sink,n,lens", [
    (6, 2, 64, 32, 5, 7, 0, 300, [300, 211]),          # R = 15 rows, D 64, pages of 32
    (16, 2, 128, 16, 40, 7, 3, 700, [700, 517]),       # R = 320: two row slabs
    (8, 2, 128, 16, 32, 1, 0, 400, [400, 33]),         # no pooling; one earlier position
    (8, 2, 128, 16, 32, 4, 0, 400, [400, 100]),        # even kernel: window j-2 .. j+2
    (8, 2, 128, 16, 32, 7, 500, 400, [400, 390]),      # every earlier position a sink
    (8, 2, 128, 16, 1, 7, 0, 257, [257, 129]),         # a single window query
    (4, 4, 128, 16, 16, 7, 0, 1100, [1100, 1000]),     # G = 1
])
def test_snapkv_scores_shapes(Hq, Hkv, D, P, w, kappa, n_sink, n, lens):
    cfg = dataclasses.replace(SMALL, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P,
                              window=w, pool_kernel=kappa, n_sink=n_sink, prompt=n)
    x = W.snapkv_inputs(cfg, 11, device="cuda", steps=1)
    kv, _ = _cache(cfg, x, lens)
    scores = _scores(cfg, kv, x)
    for b in range(2):
        for h in range(Hkv):
            _, s = _oracle_pooled(cfg, x, b, h, lens[b], w, kappa, n_sink)
            _check_scores(scores[b, h], s, lens[b], w)


def test_snapkv_short_prompts_write_nothing():
    cfg = SMALL
    x = W.snapkv_inputs(cfg, 3, device="cuda", prompt=64, steps=1)
    kv, _ = _cache(cfg, x, [32, 5])       # L = w and L < w
    scores = _scores(cfg, kv, x)
    assert bool((scores == SENTINEL).all())


# Capacities above 8192 slots compact through the kept-slot list path.
@pytest.mark.parametrize("prompt,lens,budget,n_sink", [(2048, [2048, 1543], 512, 0),
                                                       (2048, [2048, 400], 512, 4),
                                                       (9000, [9000, 8500], 1024, 0)])
def test_snapkv_retention_and_decode(prompt, lens, budget, n_sink):
    cfg = dataclasses.replace(SMALL, prompt=prompt)
    w, G = cfg.window, cfg.group
    x = W.snapkv_inputs(cfg, W.config_seed(SMALL.name), device="cuda", steps=1)
    kv, slot_pos = _cache(cfg, x, lens)
    cap = kv.capacity
    scores = _scores(cfg, kv, x, n_sink=n_sink)
    sp.sp_h2o_evict_compact(kv, scores, slot_pos, cap, budget, w,
                            sp.workspace(sp.SP_OP_H2O_EVICT, kv, budget))
    # one decode step over the retained slots
    B, H = kv.batch, kv.num_kv_heads
    pos_new = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sp.sp_build_page_meta(kv, x["k_new"][0][:, None].contiguous(), x["v_new"][0][:, None].contiguous(),
                          1, None, pos_new, slot_pos, cap)
    q = x["q"][0].contiguous()
    out = torch.empty(B, kv.num_q_heads, cfg.head_dim, device="cuda")
    lse = torch.empty(B, kv.num_q_heads, device="cuda")
    scale = W.default_scale(cfg.head_dim)
    sp.sp_sparse_decode_attn(kv, q, None, 0, scale, out, lse, ws=sp.workspace(sp.SP_OP_DECODE_ATTN, kv, 0))
    torch.cuda.synchronize()
    for b in range(B):
        n = lens[b]
        kept = min(n, budget)
        assert int(kv.seq_lens[b]) == kept + 1
        for h in range(H):
            _, s = _oracle_pooled(cfg, x, b, h, n, w, cfg.pool_kernel, n_sink)
            pos = slot_pos[b, h, :kept].cpu().numpy()
            _check_retained(pos, s, n, budget, w, n_sink)
            keys = torch.cat([x["keys"][b, h].cpu()[pos], x["k_new"][0, b, h][None].cpu()])
            vals = torch.cat([x["values"][b, h].cpu()[pos], x["v_new"][0, b, h][None].cpu()])
            for a in range(h * G, (h + 1) * G):
                o, l, _, _ = attend(f64(q[b, a]), f64(keys), f64(vals), scale)
                np.testing.assert_allclose(f64(out[b, a]), o, rtol=0, atol=2e-3)
                assert abs(float(lse[b, a]) - l) <= 2e-3


def test_snapkv_full_size_sampled_units():
    """Scores, then the compaction to the 8,192-slot budget, at the full
    workload size; checked on sampled (sequence, KV head) units."""
    name = "snapkv_qwen3_30b_a3b_b4_prompt128k_bud8k"
    cfg = W.CONFIGS[name]
    x = W.snapkv_inputs(cfg, W.config_seed(name), device="cuda")
    kv, slot_pos = _cache(cfg, x)
    scores = _scores(cfg, kv, x)
    n = x["prompt"]
    pooled = {}
    for (b, h) in [(0, 0), (3, 2)]:
        _, s = _oracle_pooled(cfg, x, b, h, n, cfg.window, cfg.pool_kernel, cfg.n_sink)
        _check_scores(scores[b, h], s, n, cfg.window)
        pooled[(b, h)] = s
    cap = kv.capacity
    sp.sp_h2o_evict_compact(kv, scores, slot_pos, cap, cfg.budget, cfg.window,
                            sp.workspace(sp.SP_OP_H2O_EVICT, kv, cfg.budget))
    torch.cuda.synchronize()
    assert kv.seq_lens.tolist() == [cfg.budget] * kv.batch
    for (b, h), s in pooled.items():
        pos = slot_pos[b, h, :cfg.budget].cpu().numpy()
        _check_retained(pos, s, n, cfg.budget, cfg.window, cfg.n_sink)
        kk, vv = sp.read_slots(kv, b, h, cfg.budget)
        assert torch.equal(kk.cpu(), x["keys"][b, h].cpu()[pos])
        assert torch.equal(vv.cpu(), x["values"][b, h].cpu()[pos])
