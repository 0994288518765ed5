#!/usr/bin/env python3
"""Sparse decode attention on one MI355X: decode-attention tokens/s and
achieved HBM GB/s against the 8 TB/s peak.

A step is one pass of the hot path over one batch of synthetic input:
  Quest workloads:   append + page-summary fold -> bound scoring + top-k ->
                     sparse split-K attention over the selected pages;
  H2O workload:      append -> dense attention with logits -> score
                     accumulation -> eviction with compaction;
  evicted workload:  append -> dense attention over the retained slots.
The headline line is the Llama-3-8B-shaped Quest layer (batch 16, 32/8 heads,
head_dim 128, 32K context, 16-token pages, 128 pages per KV head, bf16).

Inputs are seeded Gaussian tensors generated on the GPU and resident in HBM
before the timed region.  Every timed step is preceded by a 1 GiB write that
evicts the 256 MB Infinity Cache, so the bytes come from HBM; the flush is
outside the per-call HIP-event intervals that make up the step time.

Prints ONE JSON line.  `--gpus N` with N > 1 exits: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import kv_cache_selection_sp_amd as sp  # noqa: E402
import workloads as W  # noqa: E402

PEAK_HBM = 8.0e12          # MI355X HBM3E, bytes/s
HEADLINE = "quest_llama3_8b_b16_ctx32k"


def esize(dt):
    return torch.tensor([], dtype=dt).element_size()


class Flusher:
    """Writes 1 GiB so the next kernel finds neither L2 nor the Infinity Cache warm."""

    def __init__(self, dev):
        self.buf = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def __call__(self):
        self.buf.fill_(1.0)


# ----------------------------------------------------------------- workloads
class QuestRun:
    calls = ("append", "select", "attend")

    def __init__(self, cfg: W.QuestConfig, dev="cuda", context=None, batch=None):
        self.cfg = cfg
        x = W.quest_inputs(cfg, W.config_seed(cfg.name), device=dev, context=context, batch=batch)
        self.x = x
        B = x["batch"]
        dt = W.torch_dtype(cfg.dtype)
        self.kv = sp.PagedKV.allocate(B, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                                      cfg.page_size, x["max_pages"], x["num_blocks"], dt,
                                      x["block_table"], dev)
        self.meta = self.kv.new_meta()
        sp.sp_build_page_meta(self.kv, x["keys"].permute(0, 2, 1, 3).contiguous(),
                              x["values"].permute(0, 2, 1, 3).contiguous(), x["context"], self.meta)
        self.k = cfg.top_k
        self.sel = torch.empty(B, cfg.num_kv_heads, self.k, dtype=torch.int32, device=dev)
        self.ws_sel = sp.workspace(sp.SP_OP_SELECT_PAGES, self.kv, self.k)
        self.ws_attn = sp.workspace(sp.SP_OP_DECODE_ATTN, self.kv, self.k)
        self.out = torch.empty(B, cfg.num_q_heads, cfg.head_dim, device=dev)
        self.lse = torch.empty(B, cfg.num_q_heads, device=dev)
        self.scale = W.default_scale(cfg.head_dim)
        self.k_step = [x["k_new"][s][:, None].contiguous() for s in range(cfg.steps)]
        self.v_step = [x["v_new"][s][:, None].contiguous() for s in range(cfg.steps)]
        self.q_step = [x["q"][s].contiguous() for s in range(cfg.steps)]
        self.B = B
        self.L0 = x["context"]
        torch.cuda.synchronize()

    def run_call(self, name, s):
        s %= self.cfg.steps
        if name == "append":
            sp.sp_build_page_meta(self.kv, self.k_step[s], self.v_step[s], 1, self.meta)
        elif name == "select":
            sp.sp_select_pages(self.kv, self.q_step[s], self.meta, self.k, self.sel, None, self.ws_sel)
        else:
            sp.sp_sparse_decode_attn(self.kv, self.q_step[s], self.sel, self.k, self.scale,
                                     self.out, self.lse, ws=self.ws_attn)

    def tokens_per_step(self):
        return self.B

    def bytes_per_call(self, L):
        """Algorithmic HBM bytes of each call at context L (after the append)."""
        c = self.cfg
        e = esize(W.torch_dtype(c.dtype))
        P, D, H, Hq, B = c.page_size, c.head_dim, c.num_kv_heads, c.num_q_heads, self.B
        n_pages = math.ceil(L / P)
        sel_pages = min(self.k, n_pages)
        append = B * H * D * e * 2 * 2 + B * H * 2 * D * e * 2      # new K,V read+write, meta RMW
        select = (B * H * n_pages * 2 * D * e                       # page summaries
                  + B * Hq * D * e                                  # q
                  + 2 * B * H * n_pages * 4                         # scores write + read
                  + B * H * self.k * 4)
        attend = (B * H * sel_pages * P * D * e * 2                 # selected K and V
                  + B * Hq * D * e + B * Hq * (D + 1) * 4 + B * H * self.k * 4)
        return {"append": append, "select": select, "attend": attend}

    def dominant(self):
        return "attend"

    def dominant_unit_bytes(self, L):
        """Selected-KV bytes per launch of the attention kernel."""
        c = self.cfg
        e = esize(W.torch_dtype(c.dtype))
        sel_pages = min(self.k, math.ceil(L / c.page_size))
        return self.B * c.num_kv_heads * sel_pages * c.page_size * c.head_dim * e * 2


class H2ORun:
    calls = ("append", "attend", "accumulate", "evict")

    def __init__(self, cfg: W.H2OConfig, dev="cuda", batch=None):
        self.cfg = cfg
        x = W.h2o_inputs(cfg, W.config_seed(cfg.name), device=dev, batch=batch)
        self.x = x
        B = x["batch"]
        dt = W.torch_dtype(cfg.dtype)
        self.kv = sp.PagedKV.allocate(B, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                                      cfg.page_size, x["max_pages"], x["num_blocks"], dt,
                                      x["block_table"], dev)
        self.cap = self.kv.capacity
        self.scores = torch.zeros(B, cfg.num_kv_heads, self.cap, device=dev)
        self.slot_pos = torch.zeros(B, cfg.num_kv_heads, self.cap, dtype=torch.int32, device=dev)
        n = x["prompt"]
        sp.sp_build_page_meta(self.kv, x["keys"].permute(0, 2, 1, 3).contiguous(),
                              x["values"].permute(0, 2, 1, 3).contiguous(), n, None, None,
                              self.slot_pos, self.cap)
        self.scores[:, :, :n] = x["prompt_scores"]
        # prompt compaction to the budget (outside the timed decode steps)
        sp.sp_h2o_evict_compact(self.kv, self.scores, self.slot_pos, self.cap, cfg.budget,
                                cfg.recent_window)
        self.out = torch.empty(B, cfg.num_q_heads, cfg.head_dim, device=dev)
        self.lse = torch.empty(B, cfg.num_q_heads, device=dev)
        self.logits = torch.empty(B, cfg.num_q_heads, self.cap, device=dev)
        self.ws = sp.workspace(sp.SP_OP_DECODE_ATTN, self.kv, 0)
        self.scale = W.default_scale(cfg.head_dim)
        S = x["steps"]
        self.k_step = [x["k_new"][s][:, None].contiguous() for s in range(S)]
        self.v_step = [x["v_new"][s][:, None].contiguous() for s in range(S)]
        self.q_step = [x["q"][s].contiguous() for s in range(S)]
        self.pos = [torch.full((B,), n + s, dtype=torch.int32, device=dev) for s in range(S)]
        self.B = B
        self.S = S
        torch.cuda.synchronize()

    def run_call(self, name, s):
        s %= self.S
        c = self.cfg
        if name == "append":
            sp.sp_build_page_meta(self.kv, self.k_step[s], self.v_step[s], 1, None, self.pos[s],
                                  self.slot_pos, self.cap)
        elif name == "attend":
            sp.sp_sparse_decode_attn(self.kv, self.q_step[s], None, 0, self.scale, self.out,
                                     self.lse, self.logits, self.cap, self.ws)
        elif name == "accumulate":
            sp.sp_h2o_accumulate(self.kv, self.logits, self.lse, self.cap, 1, self.scores, self.cap)
        else:
            sp.sp_h2o_evict_compact(self.kv, self.scores, self.slot_pos, self.cap, c.budget,
                                    c.recent_window)

    def tokens_per_step(self):
        return self.B

    def bytes_per_call(self, L=None):
        c = self.cfg
        e = esize(W.torch_dtype(c.dtype))
        D, H, Hq, B = c.head_dim, c.num_kv_heads, c.num_q_heads, self.B
        n = c.budget + 1
        append = B * H * D * e * 2 * 2 + B * H * 4
        attend = B * H * n * D * e * 2 + B * Hq * D * e + B * Hq * n * 4 + B * Hq * (D + 1) * 4
        accumulate = B * Hq * n * 4 + B * Hq * 4 + 2 * B * H * n * 4
        # typical step: the token leaving the window is evicted, the window moves down
        moved = c.recent_window
        evict = B * H * n * 4 + B * H * moved * (2 * D * e + 8) * 2
        return {"append": append, "attend": attend, "accumulate": accumulate, "evict": evict}

    def dominant(self):
        return "attend"

    def dominant_unit_bytes(self, L=None):
        c = self.cfg
        e = esize(W.torch_dtype(c.dtype))
        return self.B * c.num_kv_heads * (c.budget + 1) * c.head_dim * e * 2


class EvictedRun:
    calls = ("append", "attend")

    def __init__(self, cfg: W.EvictedConfig, dev="cuda", batch=None):
        self.cfg = cfg
        x = W.evicted_inputs(cfg, W.config_seed(cfg.name), device=dev, batch=batch)
        self.x = x
        B = x["batch"]
        dt = W.torch_dtype(cfg.dtype)
        self.kv = sp.PagedKV.allocate(B, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                                      cfg.page_size, x["max_pages"], x["num_blocks"], dt,
                                      x["block_table"], dev)
        self.cap = self.kv.capacity
        self.slot_pos = torch.full((B, cfg.num_kv_heads, self.cap), -1, dtype=torch.int32, device=dev)
        sp.sp_build_page_meta(self.kv, x["keys"].permute(0, 2, 1, 3).contiguous(),
                              x["values"].permute(0, 2, 1, 3).contiguous(), cfg.max_len, None)
        self.kv.seq_lens.copy_(x["lens"])
        self.slot_pos[:, :, :cfg.max_len] = x["positions"]
        self.lens0 = x["lens"].clone()
        self.out = torch.empty(B, cfg.num_q_heads, cfg.head_dim, device=dev)
        self.lse = torch.empty(B, cfg.num_q_heads, device=dev)
        self.ws = sp.workspace(sp.SP_OP_DECODE_ATTN, self.kv, 0)
        self.scale = W.default_scale(cfg.head_dim)
        S = x["steps"]
        self.k_step = [x["k_new"][s][:, None].contiguous() for s in range(S)]
        self.v_step = [x["v_new"][s][:, None].contiguous() for s in range(S)]
        self.q_step = [x["q"][s].contiguous() for s in range(S)]
        self.pos = [torch.full((B,), x["source_len"] + s, dtype=torch.int32, device=dev)
                    for s in range(S)]
        self.B, self.S = B, S
        self.total_len = int(x["lens"].sum())
        torch.cuda.synchronize()

    def run_call(self, name, s):
        if s > 0 and s % self.S == 0:
            self.kv.seq_lens.copy_(self.lens0)          # wrap: back to the initial lengths
        s %= self.S
        if name == "append":
            sp.sp_build_page_meta(self.kv, self.k_step[s], self.v_step[s], 1, None, self.pos[s],
                                  self.slot_pos, self.cap)
        else:
            sp.sp_sparse_decode_attn(self.kv, self.q_step[s], None, 0, self.scale, self.out,
                                     self.lse, ws=self.ws)

    def tokens_per_step(self):
        return self.B

    def bytes_per_call(self, L=None):
        c = self.cfg
        e = esize(W.torch_dtype(c.dtype))
        D, H, Hq, B = c.head_dim, c.num_kv_heads, c.num_q_heads, self.B
        toks = self.total_len + B * (self.S // 2)
        append = B * H * D * e * 2 * 2 + B * H * 4
        attend = toks * H * D * e * 2 + B * Hq * D * e + B * Hq * (D + 1) * 4
        return {"append": append, "attend": attend}

    def dominant(self):
        return "attend"

    def dominant_unit_bytes(self, L=None):
        c = self.cfg
        e = esize(W.torch_dtype(c.dtype))
        return (self.total_len + self.B * (self.S // 2)) * c.num_kv_heads * c.head_dim * e * 2


def make_run(name, dev="cuda"):
    cfg = W.CONFIGS[name]
    if isinstance(cfg, W.QuestConfig):
        return QuestRun(cfg, dev)
    if isinstance(cfg, W.H2OConfig):
        return H2ORun(cfg, dev)
    return EvictedRun(cfg, dev)


# ----------------------------------------------------------------- timing
def time_run(run, steps, warmup, cold=True):
    """Per-call HIP-event durations over `steps` timed steps (after `warmup`).
    Returns dict(call -> list of seconds) and the wall time of the timed loop."""
    dev = run.kv.k_pool.device
    flush = Flusher(dev) if cold else None
    for s in range(warmup):
        for c in run.calls:
            run.run_call(c, s)
    torch.cuda.synchronize()
    ev = []
    t0 = time.perf_counter()
    for s in range(warmup, warmup + steps):
        if flush:
            flush()
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(len(run.calls) + 1)]
        marks[0].record()
        for i, c in enumerate(run.calls):
            run.run_call(c, s)
            marks[i + 1].record()
        ev.append(marks)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {c: [] for c in run.calls}
    for marks in ev:
        for i, c in enumerate(run.calls):
            per[c].append(marks[i].elapsed_time(marks[i + 1]) * 1e-3)
    return per, wall


def summarize(run, per, steps, L_mid=None):
    step_s = sum(sum(v) for v in per.values()) / steps
    avg = {c: sum(v) / len(v) for c, v in per.items()}
    bytes_call = run.bytes_per_call(L_mid) if L_mid is not None else run.bytes_per_call()
    all_bytes = sum(bytes_call.values())
    dom = run.dominant()
    unit = run.dominant_unit_bytes(L_mid) if L_mid is not None else run.dominant_unit_bytes()
    achieved = unit / avg[dom]
    return dict(
        tokens_per_s=run.tokens_per_step() / step_s,
        ms_per_step=step_s * 1e3,
        call_us={c: round(v * 1e6, 2) for c, v in avg.items()},
        all_bytes_per_step=all_bytes,
        all_bytes_GBps=all_bytes / step_s / 1e9,
        roofline=dict(bound="hbm", achieved=achieved / 1e9, peak=PEAK_HBM / 1e9, unit="GB/s",
                      frac=achieved / PEAK_HBM, traffic=None, kernel=dom,
                      bytes_per_launch=unit),
    )


# ----------------------------------------------------------------- CPU baseline
def cpu_baseline(run, budget_s=15.0):
    """The fp64 oracle on a bounded sample of the headline workload: whole
    (sequence, KV head) units of one decode step at full context, scaled to
    the batch."""
    import numpy as np
    from oracle import quest_decode_head
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    cfg = run.cfg
    x = run.x
    G, P = cfg.group, cfg.page_size
    units = [(b, h) for b in range(run.B) for h in range(cfg.num_kv_heads)]
    done = 0
    t0 = time.perf_counter()
    for (b, h) in units:
        keys = torch.cat([x["keys"][b, h], x["k_new"][0, b, h][None]]).cpu()
        vals = torch.cat([x["values"][b, h], x["v_new"][0, b, h][None]]).cpu()
        qs = x["q"][0, b, h * G:(h + 1) * G].cpu()
        t1 = time.perf_counter()
        quest_decode_head(qs, keys, vals, P, cfg.top_k, W.default_scale(cfg.head_dim))
        done += 1
        if time.perf_counter() - t0 > budget_s and done >= 2:
            break
        del t1
    el = time.perf_counter() - t0
    per_unit = el / done
    step_s = per_unit * len(units)
    return dict(value=run.B / step_s, unit="tokens/s", cores=cores, kind="oracle",
                threads=blas_threads,
                sample=f"{done} of {len(units)} (sequence, KV head) units of one decode step at "
                       f"full context (fp64 numpy oracle incl. its tensor copies), scaled to the batch",
                seconds=round(el, 2))


# ----------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--config", default=HEADLINE, choices=list(W.CONFIGS))
    ap.add_argument("--secondary", default="quest_gqa8_b4_ctx128k,h2o_qwen3_8b_b32_prompt8k_bud1k,"
                                           "evicted_b256_len512to2048",
                    help="comma-separated extra workloads reported under 'secondary' ('' for none)")
    ap.add_argument("--warm", action="store_true", help="skip the cache flush between steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU: this build has no multi-GPU path "
              "(the design note on sharding is in DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    sp.load()
    dev = "cuda"

    run = make_run(args.config, dev)
    per, wall = time_run(run, args.steps, args.warmup, cold=not args.warm)
    L_mid = None
    if isinstance(run, QuestRun):
        L_mid = run.L0 + args.warmup + args.steps // 2
    res = summarize(run, per, args.steps, L_mid)
    cfg = run.cfg

    secondary = {}
    for name in [n for n in args.secondary.split(",") if n and n != args.config]:
        r2 = make_run(name, dev)
        st = min(args.steps, W.CONFIGS[name].steps)
        p2, _ = time_run(r2, st, min(args.warmup, 2), cold=not args.warm)
        Lm = r2.L0 + 2 + st // 2 if isinstance(r2, QuestRun) else None
        s2 = summarize(r2, p2, st, Lm)
        s2["steps"] = st
        secondary[name] = s2
        del r2
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline and isinstance(run, QuestRun):
        cpu = cpu_baseline(run, args.cpu_seconds)

    line = {
        "metric": "sparse decode-attn tokens/sec/GPU and achieved HBM GB/s vs peak",
        "value": res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Gaussian K/V/q, no model weights)",
        "config": {"workload": cfg.name, "batch": run.B, "q_heads": cfg.num_q_heads,
                   "kv_heads": cfg.num_kv_heads, "head_dim": cfg.head_dim,
                   "context": getattr(cfg, "context", None), "page_size": cfg.page_size,
                   "top_k_pages": getattr(cfg, "top_k", None), "layers": 1,
                   "cache": "warm" if args.warm else "cold (1 GiB flush before each step)"},
        "call_us": res["call_us"],
        "all_bytes_GBps": res["all_bytes_GBps"],
        "all_bytes_frac": res["all_bytes_GBps"] * 1e9 / PEAK_HBM,
        "wall_s_timed_loop": wall,
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
