"""Helpers for the GPU parity tests: build caches through the library's own
append call, run steps, and compare with the oracle under the agreed rules.

Comparison rules:
  * floating outputs: max-abs error <= 2e-3 for bf16 inputs, <= 1e-5 for fp32
    inputs (fp32 accumulation on the GPU, fp64 in the oracle);
  * selected page sets / retained slots: bit-exact, except candidates whose
    oracle score lies within 1e-5 * max(|cutoff|, 1) of the cutoff (the k-th
    largest score); the set size must still be exact;
  * attention is checked on the GPU's own selection once it passed the set rule.
"""
from __future__ import annotations

import numpy as np
import torch

import kv_cache_selection_sp_amd as sp
import workloads as W

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-3}


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def new_cache(B, Hq, Hkv, D, P, max_pages, dtype, block_table, num_blocks=None, device="cuda"):
    nb = num_blocks if num_blocks is not None else int(block_table.max()) + 1
    return sp.PagedKV.allocate(B, Hq, Hkv, D, P, max_pages, nb, dtype, block_table, device)


def bulk_append(kv: sp.PagedKV, keys: torch.Tensor, values: torch.Tensor, meta=None,
                pos_new=None, slot_pos=None, slot_cap=0):
    """keys/values [B][H_kv][n][D] (logical order) -> appended through the library."""
    kn = keys.permute(0, 2, 1, 3).contiguous()
    vn = values.permute(0, 2, 1, 3).contiguous()
    sp.sp_build_page_meta(kv, kn, vn, kn.shape[1], meta, pos_new, slot_pos, slot_cap)


def quest_cache(cfg: W.QuestConfig, seed: int, context: int, batch: int, device="cuda"):
    x = W.quest_inputs(cfg, seed, device=device, context=context, batch=batch)
    kv = new_cache(batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size,
                   x["max_pages"], W.torch_dtype(cfg.dtype), x["block_table"],
                   num_blocks=x["num_blocks"], device=device)
    meta = kv.new_meta()
    bulk_append(kv, x["keys"], x["values"], meta)
    return x, kv, meta


def quest_gpu_step(kv, meta, x, s, top_k, scale, with_scores=True):
    """Append step s's token, select pages, attend.  Returns sel, scores, out, lse."""
    B, H, D = kv.batch, kv.num_kv_heads, kv.head_dim
    dev = kv.k_pool.device
    sp.sp_build_page_meta(kv, x["k_new"][s][:, None].contiguous(),
                          x["v_new"][s][:, None].contiguous(), 1, meta)
    sel = torch.empty(B, H, top_k, dtype=torch.int32, device=dev)
    scores = torch.empty(B, H, kv.max_pages, dtype=torch.float32, device=dev) if with_scores else None
    ws_sel = sp.workspace(sp.SP_OP_SELECT_PAGES, kv, top_k)
    q = x["q"][s].contiguous()
    sp.sp_select_pages(kv, q, meta, top_k, sel, scores, ws_sel)
    out = torch.empty(B, kv.num_q_heads, D, dtype=torch.float32, device=dev)
    lse = torch.empty(B, kv.num_q_heads, dtype=torch.float32, device=dev)
    ws = sp.workspace(sp.SP_OP_DECODE_ATTN, kv, top_k)
    sp.sp_sparse_decode_attn(kv, q, sel, top_k, scale, out, lse, ws=ws)
    return sel, scores, out, lse


def logical_kv(x, b, h, s):
    """Keys/values of (b, h) after appending steps 0..s, on the CPU."""
    k = torch.cat([x["keys"][b, h], x["k_new"][: s + 1, b, h]]).cpu()
    v = torch.cat([x["values"][b, h], x["v_new"][: s + 1, b, h]]).cpu()
    return k, v


def check_selection(got_row, oracle_scores, k):
    """got_row: GPU sel_pages row (length k); oracle_scores: fp64 [N_p]."""
    S = np.asarray(oracle_scores)
    N = len(S)
    got = [int(v) for v in got_row]
    n_sel = min(k, N)
    assert got[n_sel:] == [-1] * (k - n_sel), "padding"
    chosen = got[:n_sel]
    assert chosen == sorted(set(chosen)), "ascending, distinct"
    assert all(0 <= p < N for p in chosen), "in range"
    if k >= N:
        assert chosen == list(range(N))
        return 0
    cut = np.sort(S)[::-1][k - 1]
    tol = 1e-5 * max(abs(cut), 1.0)
    must = {p for p in range(N) if S[p] > cut + tol}
    never = {p for p in range(N) if S[p] < cut - tol}
    cs = set(chosen)
    assert must <= cs, f"missing pages {sorted(must - cs)[:8]}"
    assert not (never & cs), f"wrong pages {sorted(never & cs)[:8]}"
    return len(cs) - len(must)          # how many came from the tie band


def score_scale(qs, mins, maxs):
    """Sum of |terms| of the group bound per page: the natural error scale of
    an fp32 evaluation of S_h(p)."""
    qa = np.abs(qs).sum(axis=0)
    return np.maximum(np.abs(mins), np.abs(maxs)) @ qa


def check_quest_unit(x, kv_cfg, b, h, s, sel_row, out_bh, lse_bh, scores_row, top_k, scale, dtype,
                     n_sink=0, n_recent=0):
    """Compare one (sequence, KV head) of a Quest step with the oracle (forced
    sink and recent pages rank above every scored page)."""
    from oracle import quest_decode_head, attend
    from oracle.quest import forced_pages
    G = kv_cfg["G"]
    P = kv_cfg["P"]
    keys, values = logical_kv(x, b, h, s)
    qs = f64(x["q"][s, b, h * G:(h + 1) * G])
    r = quest_decode_head(qs, keys, values, P, top_k, scale, n_sink, n_recent)
    N = len(r["scores"])
    if scores_row is not None:
        err = np.abs(f64(scores_row[:N]) - r["scores"])
        assert np.all(err <= 1e-5 * score_scale(qs, r["mins"], r["maxs"]) + 1e-30), err.max()
        assert bool(torch.isneginf(scores_row[N:]).all())
    rank = np.array(r["scores"], dtype=np.float64)
    rank[forced_pages(N, n_sink, n_recent)] = np.inf
    check_selection(sel_row.cpu(), rank, top_k)
    # attention over the GPU's own selection
    pages = [int(p) for p in sel_row.cpu() if p >= 0]
    L = keys.shape[0]
    toks = np.concatenate([np.arange(p * P, min(L, (p + 1) * P)) for p in pages])
    kk, vv = f64(keys)[toks], f64(values)[toks]
    tol = TOL[dtype]
    for a in range(G):
        o, l, _, _ = attend(qs[a], kk, vv, scale)
        np.testing.assert_allclose(f64(out_bh[a]), o, rtol=0, atol=tol)
        assert abs(float(lse_bh[a]) - l) <= tol, (float(lse_bh[a]), l)
