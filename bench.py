#!/usr/bin/env python3
"""Sparse decode attention on one MI355X: decode-attention tokens/s and
achieved HBM GB/s against the 8 TB/s peak.

A step is one pass of the hot path over one batch of synthetic input:
  Quest workloads:   append + page-summary fold -> bound scoring + top-k ->
                     sparse split-K attention over the selected pages, in one
                     launch (sp_quest_decode_step); the "_two_launch" lines run
                     the same step as sp_append_select_pages followed by
                     sp_sparse_decode_attn, so the attention kernel's own
                     roofline is reported too;
  H2O workload:      append -> dense attention with logits -> score
                     accumulation -> eviction with compaction;
  evicted workload:  append -> dense attention over the retained slots;
  SnapKV workload:   window scoring + pooling of every prompt position ->
                     compaction of the prompt cache to the budget (its value
                     counts prompt tokens selected per second);
  H2O prefill:       per prompt chunk, append -> chunk attention probabilities
                     added to the scores -> eviction to the budget (prompt
                     tokens prefilled per second);
  OmniKV:            observation-layer token scores + top-b selection ->
                     the sparse layer's attention over the reused positions
                     of its own cache (decode tokens per second).
The headline line is the Llama-3-8B-shaped Quest layer (batch 16, 32/8 heads,
head_dim 128, 32K context, 16-token pages, 128 pages per KV head, bf16).

Inputs are seeded Gaussian tensors generated on the GPU and resident in HBM
before any timing.  Each step's query and new key/value are copied into
address-stable buffers before the step (as a serving engine does before a
graph replay), and every timed step is preceded by a 1 GiB write that evicts
L2 and the 256 MB Infinity Cache, so the step's bytes come from HBM.

Protocol (after the pages' measurement protocol): `--warmup` untimed steps
stand for the discarded workload, then three windows of `--steps` steps each;
`ms_per_step` is the median of the windows' mean step times, which are listed
in `window_ms_per_step`.

Timings, all with HIP events on the stream the library launches on (torch's
current stream):
  * per step, the step's calls launched back to back: the step time behind
    `value` and `ms_per_step` (one event pair around the whole step, so the
    gaps between its kernels count);
  * per call, from events between the calls of the same steps: a decode call
    is a single kernel, so these are kernel durations (the dominant call's
    gives roofline.achieved);
  * the same step captured once into a HIP graph and replayed, reported as
    `graph_ms_per_step`.  On this platform a replay adds several microseconds
    per launch to a step of a few long kernels, so the eager step is the
    faster way to run it and is the one `value` reports.

cpu_baseline: the fp64 oracle on the host cores in the same run, over a
bounded sample of the headline workload (whole (sequence, KV head) units at
full context), at every core and at one thread; the 128K Quest, H2O and
evicted lines carry their own oracle timings over stated subsets.

Prints ONE JSON line.  `--gpus N` with N > 1 exits: the path runs on one GPU.
`--copy-calibration` instead runs a plain 1 GiB device copy (the known-size
kernel that scales the HBM byte counters) and prints its timing.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import kv_cache_selection_sp_amd as sp  # noqa: E402
import workloads as W  # noqa: E402

PEAK_HBM = 8.0e12          # MI355X HBM3E, bytes/s
PEAK_MFMA_BF16 = 2.5e15    # MI355X dense bf16 MFMA, flop/s
HEADLINE = "quest_llama3_8b_b16_ctx32k"
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
CSRC = os.path.join(ROOT, "kv_cache_selection_sp_amd", "csrc")


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
    """A Quest decode step.  Single-launch form (default): sp_quest_decode_step
    appends the decode token, selects the pages and attends in one launch.
    Two-launch form: sp_append_select_pages, then sp_sparse_decode_attn."""

    def __init__(self, cfg: W.QuestConfig, dev, spare_tokens: int, variant=None, fused=True):
        self.cfg = cfg
        # (name, n_sink, n_recent, group_reduce) of a selection variant, or None
        self.variant = variant
        self.fused = fused
        if fused:
            self.calls = ("step",)
            self.dominant = "step"
            self.dominant_kernel = "sp_quest_decode_step (quest_step_kernel: append + select + attend)"
        else:
            self.calls = ("append_select", "attend")
            self.dominant = "attend"
            self.dominant_kernel = "sp_sparse_decode_attn (attn_kernel)"
        x = W.quest_inputs(cfg, W.config_seed(cfg.name), device=dev, spare_tokens=spare_tokens)
        self.x = x
        B = x["batch"]
        dt = W.torch_dtype(cfg.dtype)
        self.kv = sp.PagedKV.allocate(B, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                                      cfg.page_size, x["max_pages"], x["num_blocks"], dt,
                                      x["block_table"], dev)
        self.meta = self.kv.new_meta()
        sp.sp_build_page_meta(self.kv, x["keys"].permute(0, 2, 1, 3).contiguous(),
                              x["values"].permute(0, 2, 1, 3).contiguous(), x["context"], self.meta)
        # whether the step entry point runs as one launch here (else its two launches)
        red = variant[3] if variant is not None else sp.SP_GROUP_SUM
        self.single = fused and sp.sp_quest_step_single_launch(self.kv, red)
        if fused and not self.single:
            self.dominant_kernel = "sp_quest_decode_step (select_kernel + attn_kernel: its two-launch form)"
        self.k = cfg.top_k
        self.sel = torch.empty(B, cfg.num_kv_heads, self.k, dtype=torch.int32, device=dev)
        if fused:
            self.ws_step = sp.workspace(sp.SP_OP_QUEST_STEP, self.kv, self.k)
        else:
            self.ws_sel = sp.workspace(sp.SP_OP_SELECT_PAGES, self.kv, self.k)
            self.ws_attn = sp.workspace(sp.SP_OP_DECODE_ATTN, self.kv, self.k)
        self.out = torch.empty(B, cfg.num_q_heads, cfg.head_dim, device=dev)
        self.lse = torch.empty(B, cfg.num_q_heads, device=dev)
        self.scale = W.default_scale(cfg.head_dim)
        self.q = torch.empty_like(x["q"][0])
        self.k1 = torch.empty_like(x["k_new"][0])
        self.v1 = torch.empty_like(x["v_new"][0])
        self.kn = self.k1[:, None]
        self.vn = self.v1[:, None]
        self.B = B
        self.L = x["context"]          # host mirror of the (uniform) length
        torch.cuda.synchronize()

    def load_step(self, s):
        s %= self.cfg.steps
        self.q.copy_(self.x["q"][s])
        self.k1.copy_(self.x["k_new"][s])
        self.v1.copy_(self.x["v_new"][s])

    def call(self, name):
        _, n_sink, n_recent, red = self.variant if self.variant is not None else (None, 0, 0, sp.SP_GROUP_SUM)
        if name == "step":
            sp.sp_quest_decode_step(self.kv, self.k1, self.v1, None, None, 0, self.meta, self.q, self.k, n_sink,
                                    n_recent, red, self.scale, self.sel, None, self.out, self.lse, self.ws_step)
        elif name == "append_select":
            sp.sp_append_select_pages(self.kv, self.k1, self.v1, None, None, 0, self.meta, self.q, self.k,
                                      n_sink, n_recent, red, self.sel, None, self.ws_sel)
        else:
            sp.sp_sparse_decode_attn(self.kv, self.q, self.sel, self.k, self.scale,
                                     self.out, self.lse, ws=self.ws_attn)

    def after_step(self):
        self.L += 1

    def bytes_per_call(self):
        """Algorithmic HBM bytes of each call at the current length."""
        c = self.cfg
        e = esize(W.torch_dtype(c.dtype))
        P, D, H, Hq, B = c.page_size, c.head_dim, c.num_kv_heads, c.num_q_heads, self.B
        n_pages = math.ceil(self.L / P)
        sel_pages = min(self.k, n_pages)
        append = B * H * D * e * 2 * 2 + B * H * 2 * D * e * 2      # new K,V read+write, summary RMW
        select = (B * H * n_pages * 2 * D * e                       # page summaries
                  + B * Hq * D * e                                  # q
                  + 2 * B * H * n_pages * 4                         # scores written, read back
                  + B * H * self.k * 4)                             # selection written
        attend = (B * H * sel_pages * P * D * e * 2                 # selected K and V
                  + B * Hq * D * e + B * Hq * (D + 1) * 4 + B * H * self.k * 4)
        if self.fused:
            return {"step": append + select + attend}
        return {"append_select": append + select, "attend": attend}

    def selected_kv_bytes(self):
        """Selected-KV bytes of one step."""
        c = self.cfg
        e = esize(W.torch_dtype(c.dtype))
        sel_pages = min(self.k, math.ceil(self.L / c.page_size))
        return self.B * c.num_kv_heads * sel_pages * c.page_size * c.head_dim * e * 2

    def dominant_unit_bytes(self):
        """Algorithmic bytes per launch of the dominant kernel: the single
        launch's page summaries, selected K/V and small terms, or the
        attention kernel's selected K/V."""
        if self.fused:
            return self.bytes_per_call()["step"]
        return self.selected_kv_bytes()

    def config(self):
        c = self.cfg
        d = {"workload": c.name if self.variant is None else self.variant[0], "batch": self.B,
             "q_heads": c.num_q_heads, "kv_heads": c.num_kv_heads, "head_dim": c.head_dim,
             "context": c.context, "page_size": c.page_size, "top_k_pages": c.top_k, "layers": 1,
             "launches": "one (sp_quest_decode_step)" if self.single
             else "two (sp_quest_decode_step: select, then attention)" if self.fused
             else "two (sp_append_select_pages, sp_sparse_decode_attn)"}
        if self.variant is not None:
            _, n_sink, n_recent, red = self.variant
            d.update(sink_pages=n_sink, recent_pages=n_recent,
                     group_reduce="max" if red == sp.SP_GROUP_MAX else "sum")
        return d


class H2ORun:
    # the dense attention and the score update share one launch
    # (sp_decode_attn_accumulate), then the eviction
    calls = ("append", "attend_acc", "evict")
    dominant = "attend_acc"
    dominant_kernel = "sp_decode_attn_accumulate (attn_kernel with the score update)"

    def __init__(self, cfg: W.H2OConfig, dev, spare_tokens: int = 0):
        self.cfg = cfg
        x = W.h2o_inputs(cfg, W.config_seed(cfg.name), device=dev)
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
        # the prompt's H2O scores: its own queries' causal attention
        # probabilities, the whole prompt being one prefill chunk
        sp.sp_h2o_prefill_scores(self.kv, x["q_prompt"], n, W.default_scale(cfg.head_dim), self.scores,
                                 self.cap, sp.workspace(sp.SP_OP_H2O_PREFILL, self.kv, n))
        x.pop("q_prompt")
        # eviction workspace: per-sequence counters, so the length update
        # happens inside the eviction kernel
        self.ws_e = sp.workspace(sp.SP_OP_H2O_EVICT, self.kv, cfg.budget)
        # prompt compaction to the budget (before any timed decode step)
        sp.sp_h2o_evict_compact(self.kv, self.scores, self.slot_pos, self.cap, cfg.budget,
                                cfg.recent_window, self.ws_e)
        self.out = torch.empty(B, cfg.num_q_heads, cfg.head_dim, device=dev)
        self.lse = torch.empty(B, cfg.num_q_heads, device=dev)
        self.logits = torch.empty(B, cfg.num_q_heads, self.cap, device=dev)
        self.ws = sp.workspace(sp.SP_OP_DECODE_ATTN, self.kv, 0)
        self.scale = W.default_scale(cfg.head_dim)
        self.q = torch.empty_like(x["q"][0])
        self.kn = torch.empty_like(x["k_new"][0][:, None])
        self.vn = torch.empty_like(x["v_new"][0][:, None])
        self.pos = torch.zeros(B, dtype=torch.int32, device=dev)
        self.B = B
        self.S = x["steps"]
        self.i = n                       # logical position of the next token
        torch.cuda.synchronize()

    def load_step(self, s):
        s %= self.S
        self.q.copy_(self.x["q"][s])
        self.kn.copy_(self.x["k_new"][s][:, None])
        self.vn.copy_(self.x["v_new"][s][:, None])
        self.pos.fill_(self.i)

    def call(self, name):
        c = self.cfg
        if name == "append":
            sp.sp_build_page_meta(self.kv, self.kn, self.vn, 1, None, self.pos, self.slot_pos, self.cap)
        elif name == "attend_acc":
            sp.sp_decode_attn_accumulate(self.kv, self.q, self.scale, self.out, self.lse, self.logits,
                                         self.cap, 1, self.scores, self.cap, self.ws)
        else:
            sp.sp_h2o_evict_compact(self.kv, self.scores, self.slot_pos, self.cap, c.budget,
                                    c.recent_window, self.ws_e)

    def after_step(self):
        self.i += 1

    def bytes_per_call(self):
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
        return {"append": append, "attend_acc": attend + accumulate, "evict": evict}

    def dominant_unit_bytes(self):
        """The fused call's algorithmic bytes: K and V of every occupied slot,
        q, out, lse, the logits written and read back, the scores updated."""
        return self.bytes_per_call()["attend_acc"]

    def config(self):
        c = self.cfg
        return {"workload": c.name, "batch": self.B, "q_heads": c.num_q_heads,
                "kv_heads": c.num_kv_heads, "head_dim": c.head_dim, "prompt": c.prompt,
                "budget": c.budget, "recent_window": c.recent_window, "page_size": c.page_size,
                "layers": 1}


class EvictedRun:
    calls = ("append", "attend")
    dominant = "attend"

    def __init__(self, cfg: W.EvictedConfig, dev, spare_tokens: int = 0):
        self.cfg = cfg
        x = W.evicted_inputs(cfg, W.config_seed(cfg.name), device=dev)
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
        self.q = torch.empty_like(x["q"][0])
        self.kn = torch.empty_like(x["k_new"][0][:, None])
        self.vn = torch.empty_like(x["v_new"][0][:, None])
        self.pos = torch.zeros(B, dtype=torch.int32, device=dev)
        self.B, self.S = B, x["steps"]
        self.total0 = int(x["lens"].sum())
        self.n_app = 0                   # appends since the lengths were last reset
        torch.cuda.synchronize()

    def load_step(self, s):
        if s > 0 and s % self.S == 0:
            self.kv.seq_lens.copy_(self.lens0)          # wrap: back to the initial lengths
            self.n_app = 0
        s %= self.S
        self.q.copy_(self.x["q"][s])
        self.kn.copy_(self.x["k_new"][s][:, None])
        self.vn.copy_(self.x["v_new"][s][:, None])
        self.pos.fill_(self.x["source_len"] + s)

    def call(self, name):
        if name == "append":
            sp.sp_build_page_meta(self.kv, self.kn, self.vn, 1, None, self.pos, self.slot_pos, self.cap)
        else:
            sp.sp_sparse_decode_attn(self.kv, self.q, None, 0, self.scale, self.out, self.lse,
                                     ws=self.ws)

    def after_step(self):
        self.n_app += 1

    def _tokens(self):
        return self.total0 + self.B * self.n_app

    def bytes_per_call(self):
        c = self.cfg
        e = esize(W.torch_dtype(c.dtype))
        D, H, Hq, B = c.head_dim, c.num_kv_heads, c.num_q_heads, self.B
        append = B * H * D * e * 2 * 2 + B * H * 4
        attend = self._tokens() * H * D * e * 2 + B * Hq * D * e + B * Hq * (D + 1) * 4
        return {"append": append, "attend": attend}

    def dominant_unit_bytes(self):
        c = self.cfg
        e = esize(W.torch_dtype(c.dtype))
        return self._tokens() * c.num_kv_heads * c.head_dim * e * 2

    def config(self):
        c = self.cfg
        return {"workload": c.name, "batch": self.B, "q_heads": c.num_q_heads,
                "kv_heads": c.num_kv_heads, "head_dim": c.head_dim,
                "retained_len": [c.min_len, c.max_len], "page_size": c.page_size, "layers": 1}


class SnapKVRun:
    """SnapKV prompt selection over a batch of full prompts: window scoring +
    pooling, then compaction to the budget.  Every step starts from the same
    full prompt cache (restored before the step, outside the timed region).
    `value` for this workload counts prompt tokens selected per second."""
    calls = ("scores", "evict")
    dominant = "scores"
    dominant_kernel = "sp_snapkv_scores (snap_lse_kernel + snap_score_kernel + merge + pool)"

    def __init__(self, cfg: W.SnapKVConfig, dev, spare_tokens: int = 0):
        self.cfg = cfg
        x = W.snapkv_inputs(cfg, W.config_seed(cfg.name), device=dev)
        B = x["batch"]
        dt = W.torch_dtype(cfg.dtype)
        self.kv = sp.PagedKV.allocate(B, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                                      cfg.page_size, x["max_pages"], x["num_blocks"], dt,
                                      x["block_table"], dev)
        self.cap = self.kv.capacity
        self.n = x["prompt"]
        self.slot_pos = torch.zeros(B, cfg.num_kv_heads, self.cap, dtype=torch.int32, device=dev)
        sp.sp_build_page_meta(self.kv, x["keys"].permute(0, 2, 1, 3).contiguous(),
                              x["values"].permute(0, 2, 1, 3).contiguous(), self.n, None, None,
                              self.slot_pos, self.cap)
        self.q_obs = x["q_obs"].contiguous()
        del x
        # pristine prompt state, restored before every step
        self.k0, self.v0 = self.kv.k_pool.clone(), self.kv.v_pool.clone()
        self.pos0, self.lens0 = self.slot_pos.clone(), self.kv.seq_lens.clone()
        self.scores = torch.zeros(B, cfg.num_kv_heads, self.cap, device=dev)
        self.ws_s = sp.workspace(sp.SP_OP_SNAPKV_SCORES, self.kv, cfg.window)
        self.ws_e = sp.workspace(sp.SP_OP_H2O_EVICT, self.kv, cfg.budget)
        self.scale = W.default_scale(cfg.head_dim)
        self.B = B
        torch.cuda.synchronize()

    def prepare(self, s):
        self.kv.k_pool.copy_(self.k0)
        self.kv.v_pool.copy_(self.v0)
        self.slot_pos.copy_(self.pos0)
        self.kv.seq_lens.copy_(self.lens0)

    def load_step(self, s):
        pass

    def call(self, name):
        c = self.cfg
        if name == "scores":
            sp.sp_snapkv_scores(self.kv, self.q_obs, c.window, self.scale, c.pool_kernel, c.n_sink,
                                self.scores, self.cap, self.ws_s)
        else:
            sp.sp_h2o_evict_compact(self.kv, self.scores, self.slot_pos, self.cap, c.budget, c.window,
                                    self.ws_e)

    def after_step(self):
        pass

    def tokens_per_step(self):
        return self.B * self.n

    def bytes_per_call(self):
        c = self.cfg
        e = esize(W.torch_dtype(c.dtype))
        D, H, Hq, B, n, w = c.head_dim, c.num_kv_heads, c.num_q_heads, self.B, self.n, c.window
        kbytes = B * H * n * D * e
        # two sweeps over K (normalisers, then scores), window queries, u per
        # row slab written and read back, pooled scores written
        scores = 2 * kbytes + B * w * Hq * D * e + 2 * B * H * (n - w) * 4 + B * H * (n - w) * 4
        # scores read for the selection and the ranks; kept K, V, score and
        # position read and written
        evict = 5 * B * H * n * 4 + B * H * c.budget * (2 * D * e + 8) * 2
        return {"scores": scores, "evict": evict}

    def dominant_unit_bytes(self):
        """K bytes the two sweeps of one scoring call stream."""
        c = self.cfg
        return 2 * self.B * c.num_kv_heads * self.n * c.head_dim * esize(W.torch_dtype(c.dtype))

    def config(self):
        c = self.cfg
        return {"workload": c.name, "batch": self.B, "q_heads": c.num_q_heads,
                "kv_heads": c.num_kv_heads, "head_dim": c.head_dim, "prompt": self.n,
                "window": c.window, "pool_kernel": c.pool_kernel, "budget": c.budget,
                "page_size": c.page_size, "layers": 1}


class H2OPrefillRun:
    """H2O over whole prompts prefilled chunk by chunk: per chunk, append its
    K/V, add its queries' attention probabilities to the scores
    (sp_h2o_prefill_scores), evict to the budget.  Every step starts from an
    empty cache (lengths reset before the step, outside the timed region).
    `value` for this workload counts prompt tokens prefilled per second."""
    dominant_kernel = "sp_h2o_prefill_scores (snap_lse_kernel + snap_score_kernel + merge + accumulate)"

    def __init__(self, cfg: W.H2OPrefillConfig, dev, spare_tokens: int = 0):
        self.cfg = cfg
        x = W.h2o_prefill_inputs(cfg, W.config_seed(cfg.name), device=dev)
        B, n, C = x["batch"], x["prompt"], cfg.chunk
        dt = W.torch_dtype(cfg.dtype)
        self.kv = sp.PagedKV.allocate(B, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                                      cfg.page_size, x["max_pages"], x["num_blocks"], dt,
                                      x["block_table"], dev)
        self.cap = self.kv.capacity
        self.slot_pos = torch.zeros(B, cfg.num_kv_heads, self.cap, dtype=torch.int32, device=dev)
        self.scores = torch.zeros(B, cfg.num_kv_heads, self.cap, device=dev)
        self.chunks = []
        for c0 in range(0, n, C):
            c1 = min(n, c0 + C)
            self.chunks.append(dict(
                n=c1 - c0, L=min(c0, cfg.budget) + (c1 - c0),
                k=x["keys"][:, :, c0:c1].permute(0, 2, 1, 3).contiguous(),
                v=x["values"][:, :, c0:c1].permute(0, 2, 1, 3).contiguous(),
                q=x["q"][:, c0:c1].contiguous(),
                pos=torch.full((B,), c0, dtype=torch.int32, device=dev)))
        del x
        self.ws_s = sp.workspace(sp.SP_OP_H2O_PREFILL, self.kv, C)
        self.ws_e = sp.workspace(sp.SP_OP_H2O_EVICT, self.kv, cfg.budget)
        self.scale = W.default_scale(cfg.head_dim)
        self.B, self.n = B, n
        nc = len(self.chunks)
        self.calls = tuple(f"{op}{c}" for c in range(nc) for op in ("append", "score", "evict"))
        self.dominant = f"score{nc - 1}"
        torch.cuda.synchronize()

    def prepare(self, s):
        self.kv.seq_lens.zero_()

    def load_step(self, s):
        pass

    def call(self, name):
        c = self.cfg
        op, i = name.rstrip("0123456789"), int(name[len(name.rstrip("0123456789")):])
        ch = self.chunks[i]
        if op == "append":
            sp.sp_build_page_meta(self.kv, ch["k"], ch["v"], ch["n"], None, ch["pos"], self.slot_pos,
                                  self.cap)
        elif op == "score":
            sp.sp_h2o_prefill_scores(self.kv, ch["q"], ch["n"], self.scale, self.scores, self.cap, self.ws_s)
        else:
            sp.sp_h2o_evict_compact(self.kv, self.scores, self.slot_pos, self.cap, c.budget,
                                    c.recent_window, self.ws_e)

    def after_step(self):
        pass

    def tokens_per_step(self):
        return self.B * self.n

    def bytes_per_call(self):
        c = self.cfg
        e = esize(W.torch_dtype(c.dtype))
        D, H, Hq, B = c.head_dim, c.num_kv_heads, c.num_q_heads, self.B
        out = {}
        for i, ch in enumerate(self.chunks):
            n_q, L = ch["n"], ch["L"]
            out[f"append{i}"] = B * H * n_q * D * e * 2 * 2 + B * H * n_q * 4
            # two sweeps over the available K, the chunk's queries, scores read and written
            out[f"score{i}"] = 2 * B * H * L * D * e + B * n_q * Hq * D * e + 2 * B * H * L * 4
            out[f"evict{i}"] = 5 * B * H * L * 4 + B * H * c.budget * (2 * D * e + 8) * 2
        return out

    def dominant_flops(self):
        """MFMA flops of the last chunk's scoring: two sweeps of 2 * D flops
        per (query row, visible key) pair; query i of the chunk sees the
        retained slots and the chunk up to itself."""
        c, ch = self.cfg, self.chunks[-1]
        n_q, n_r = ch["n"], ch["L"] - ch["n"]
        pairs = c.group * (n_q * n_r + n_q * (n_q + 1) // 2)
        return 2 * 2 * c.head_dim * pairs * self.B * c.num_kv_heads

    def dominant_unit_bytes(self):
        """Available-K bytes the two sweeps of the last chunk's scoring stream."""
        c = self.cfg
        return 2 * self.B * c.num_kv_heads * self.chunks[-1]["L"] * c.head_dim * esize(W.torch_dtype(c.dtype))

    def config(self):
        c = self.cfg
        return {"workload": c.name, "batch": self.B, "q_heads": c.num_q_heads,
                "kv_heads": c.num_kv_heads, "head_dim": c.head_dim, "prompt": self.n,
                "chunk": c.chunk, "budget": c.budget, "recent_window": c.recent_window,
                "page_size": c.page_size, "layers": 1}


class OmniKVRun:
    """OmniKV decode step over two layers' caches: the observation layer's
    selection (token scores over its whole cache, top-b, pages + masks), then
    the sparse layer's attention over the reused positions of its own cache."""
    calls = ("select", "attend")
    dominant = "select"
    dominant_kernel = "sp_omnikv_select (omni_score_kernel + top-b list kernels)"

    def __init__(self, cfg: W.OmniKVConfig, dev, spare_tokens: int = 0):
        self.cfg = cfg
        x = W.omnikv_inputs(cfg, W.config_seed(cfg.name), device=dev)
        B, L = x["batch"], x["context"]
        dt = W.torch_dtype(cfg.dtype)

        def cache(k, v):
            kv = sp.PagedKV.allocate(B, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size,
                                     x["max_pages"], x["num_blocks"], dt, x["block_table"], dev)
            sp.sp_build_page_meta(kv, k.permute(0, 2, 1, 3).contiguous(), v.permute(0, 2, 1, 3).contiguous(),
                                  L, None)
            return kv
        self.kv_obs = cache(x["keys_obs"], x["values_obs"])
        self.kv = cache(x["keys"], x["values"])
        self.q_obs_all, self.q_all = x["q_obs"], x["q"]
        del x
        self.kp = min(cfg.top_b, self.kv.max_pages)
        self.pages = torch.empty(B, cfg.num_kv_heads, self.kp, dtype=torch.int32, device=dev)
        self.mask = torch.empty(B, cfg.num_kv_heads, self.kp, dtype=torch.int32, device=dev)
        self.ts = torch.empty(B, self.kv.capacity, device=dev)
        self.ws_s = sp.workspace(sp.SP_OP_OMNIKV_SELECT, self.kv_obs, cfg.top_b)
        self.ws_a = sp.workspace(sp.SP_OP_DECODE_ATTN, self.kv, self.kp)
        self.out = torch.empty(B, cfg.num_q_heads, cfg.head_dim, device=dev)
        self.lse = torch.empty(B, cfg.num_q_heads, device=dev)
        self.q_obs = torch.empty_like(self.q_obs_all[0])
        self.q = torch.empty_like(self.q_all[0])
        self.scale = W.default_scale(cfg.head_dim)
        self.B, self.L = B, L
        torch.cuda.synchronize()

    def load_step(self, s):
        s %= self.cfg.steps
        self.q_obs.copy_(self.q_obs_all[s])
        self.q.copy_(self.q_all[s])

    def call(self, name):
        if name == "select":
            sp.sp_omnikv_select(self.kv_obs, self.q_obs, self.cfg.top_b, self.pages, self.mask, self.kp,
                                self.ts, self.kv.capacity, self.ws_s)
        else:
            sp.sp_sparse_decode_attn_masked(self.kv, self.q, self.pages, self.mask, self.kp, self.scale,
                                            self.out, self.lse, self.ws_a)

    def after_step(self):
        pass

    def bytes_per_call(self):
        c = self.cfg
        e = esize(W.torch_dtype(c.dtype))
        D, H, Hq, B, L = c.head_dim, c.num_kv_heads, c.num_q_heads, self.B, self.L
        select = B * H * L * D * e + B * Hq * D * e + 6 * B * L * 4
        # at least the selected tokens' K and V; whole pages are read
        attend = B * H * c.top_b * D * e * 2 + B * Hq * D * e + B * Hq * (D + 1) * 4
        return {"select": select, "attend": attend}

    def dominant_unit_bytes(self):
        """The observation layer's K, read once by the token scoring."""
        c = self.cfg
        return self.B * c.num_kv_heads * self.L * c.head_dim * esize(W.torch_dtype(c.dtype))

    def config(self):
        c = self.cfg
        return {"workload": c.name, "batch": self.B, "q_heads": c.num_q_heads,
                "kv_heads": c.num_kv_heads, "head_dim": c.head_dim, "context": self.L,
                "top_b_tokens": c.top_b, "page_size": c.page_size, "layers": 2}


# Selection variants of the Quest workloads (same shapes and inputs): the
# pages' baseline budget of 4 sink + 32 recent + 92 selected pages, and the
# max-over-group aggregation of the page bound.
VARIANTS = {
    "quest_sink4_recent32_llama3_8b_b16_ctx32k": ("quest_llama3_8b_b16_ctx32k", 4, 32, sp.SP_GROUP_SUM),
    "quest_groupmax_gqa8_b4_ctx128k": ("quest_gqa8_b4_ctx128k", 0, 0, sp.SP_GROUP_MAX),
}


TWO_LAUNCH = "_two_launch"


def workload_names():
    quest = [n for n, c in W.CONFIGS.items() if isinstance(c, W.QuestConfig)]
    return list(W.CONFIGS) + list(VARIANTS) + [n + TWO_LAUNCH for n in quest + list(VARIANTS)]


def make_run(name, dev, spare_tokens):
    fused = not name.endswith(TWO_LAUNCH)
    base_name = name[:-len(TWO_LAUNCH)] if not fused else name
    if base_name in VARIANTS:
        base, n_sink, n_recent, red = VARIANTS[base_name]
        return QuestRun(W.CONFIGS[base], dev, spare_tokens, (name, n_sink, n_recent, red), fused=fused)
    cfg = W.CONFIGS[base_name]
    if isinstance(cfg, W.QuestConfig):
        r = QuestRun(cfg, dev, spare_tokens, fused=fused)
        if not fused:
            r.variant = (name, 0, 0, sp.SP_GROUP_SUM)
        return r
    if isinstance(cfg, W.H2OConfig):
        return H2ORun(cfg, dev)
    if isinstance(cfg, W.SnapKVConfig):
        return SnapKVRun(cfg, dev)
    if isinstance(cfg, W.H2OPrefillConfig):
        return H2OPrefillRun(cfg, dev)
    if isinstance(cfg, W.OmniKVConfig):
        return OmniKVRun(cfg, dev)
    return EvictedRun(cfg, dev)


# ----------------------------------------------------------------- timing
WINDOWS = 3


def measure(run, steps, warmup, cold=True):
    """`warmup` untimed steps, then WINDOWS windows of `steps` eager steps each
    (per-call events and the whole step's), then `steps` replays of the step
    captured into a HIP graph.  The warm-up plays the part of the discarded
    workload of the pages' protocol; the step time reported is the median of
    the windows' means."""
    dev = run.kv.k_pool.device
    flush = Flusher(dev) if cold else None
    s = 0
    prepare = getattr(run, "prepare", None)
    for _ in range(warmup):
        if prepare:
            prepare(s)
        run.load_step(s)
        for c in run.calls:
            run.call(c)
        run.after_step()
        s += 1
    torch.cuda.synchronize()
    # eager: one event pair per call; the first and last give the step
    per = {c: [] for c in run.calls}
    step_t, windows = [], []
    unit_bytes, call_bytes = [], []
    t0 = time.perf_counter()
    for _ in range(WINDOWS):
        win = []
        for _ in range(steps):
            if prepare:
                prepare(s)
            if flush:
                flush()
            run.load_step(s)
            marks = [torch.cuda.Event(enable_timing=True) for _ in range(len(run.calls) + 1)]
            marks[0].record()
            for i, c in enumerate(run.calls):
                run.call(c)
                marks[i + 1].record()
            run.after_step()
            unit_bytes.append(run.dominant_unit_bytes())
            call_bytes.append(run.bytes_per_call())
            torch.cuda.synchronize()
            for i, c in enumerate(run.calls):
                per[c].append(marks[i].elapsed_time(marks[i + 1]) * 1e-3)
            win.append(marks[0].elapsed_time(marks[-1]) * 1e-3)
            s += 1
        windows.append(statistics.mean(win))
        step_t += win
    wall = time.perf_counter() - t0
    # graph: capture the step's calls once, replay
    g = torch.cuda.CUDAGraph()
    if prepare:
        prepare(s)
    run.load_step(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for c in run.calls:
            run.call(c)
    torch.cuda.synchronize()
    graph_t = []
    torch.cuda.synchronize()
    for _ in range(steps):
        if prepare:
            prepare(s)
        if flush:
            flush()
        run.load_step(s)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        run.after_step()
        torch.cuda.synchronize()
        graph_t.append(e0.elapsed_time(e1) * 1e-3)
        s += 1
    del g
    return per, step_t, windows, graph_t, unit_bytes, call_bytes, wall


def source_hash():
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def counter_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed counter
    runs (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter on a
    plain copy of known size), or None when the kernels have changed since."""
    try:
        with open(COUNTERS) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    w = rec.get("workloads", {}).get(workload)
    if not w or rec.get("source_sha256") != source_hash():
        return None
    return w["fetch_kib"] * 1024 * rec["fetch_scale"] + w["write_kib"] * 1024 * rec["write_scale"]


def summarize(run, per, step_t, windows, graph_t, unit_bytes, call_bytes, name):
    steps = len(step_t) // len(windows)
    avg = {c: statistics.median(v) for c, v in per.items()}
    step_s = statistics.median(windows)
    graph_step_s = statistics.mean(graph_t)
    all_bytes = statistics.mean(sum(cb.values()) for cb in call_bytes)
    unit = statistics.mean(unit_bytes)
    achieved = unit / avg[run.dominant]
    if hasattr(run, "dominant_flops"):
        # compute-bound workloads: the dominant call's algorithmic MFMA flops
        flops = run.dominant_flops()
        roof = dict(bound="mfma", achieved=flops / avg[run.dominant] / 1e12, peak=PEAK_MFMA_BF16 / 1e12,
                    unit="TFLOP/s", frac=flops / avg[run.dominant] / PEAK_MFMA_BF16,
                    traffic=counter_traffic(name), kernel=run.dominant_kernel, flops_per_launch=flops,
                    hbm_GBps=achieved / 1e9)
    else:
        roof = dict(bound="hbm", achieved=achieved / 1e9, peak=PEAK_HBM / 1e9, unit="GB/s",
                    frac=achieved / PEAK_HBM, traffic=counter_traffic(name),
                    kernel=getattr(run, "dominant_kernel", "sp_sparse_decode_attn (attn_kernel)"),
                    bytes_per_launch=unit)
    if roof.get("traffic"):
        # HBM bytes from the counters over the dominant call's event time
        roof["traffic_GBps"] = roof["traffic"] / avg[run.dominant] / 1e9
    if getattr(run, "fused", False):
        # the single launch's share that is selected K/V
        kvb = run.selected_kv_bytes()
        roof["selected_kv_bytes"] = kvb
        roof["selected_kv_GBps"] = kvb / avg[run.dominant] / 1e9
    tokens = run.tokens_per_step() if hasattr(run, "tokens_per_step") else run.B
    return dict(
        tokens_per_s=tokens / step_s,
        ms_per_step=step_s * 1e3,
        graph_ms_per_step=graph_step_s * 1e3,
        call_us={c: round(v * 1e6, 2) for c, v in avg.items()},
        window_ms_per_step=[round(w * 1e3, 4) for w in windows],
        all_bytes_per_step=all_bytes,
        all_bytes_GBps=all_bytes / step_s / 1e9,
        all_bytes_frac=all_bytes / step_s / PEAK_HBM,
        roofline=roof,
        steps=steps,
    )


# ----------------------------------------------------------------- CPU baseline
def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return None


def _limit_threads(n):
    """A context that limits numpy's BLAS/OpenMP pools to n threads (no-op
    without threadpoolctl)."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=n)
    except Exception:
        import contextlib
        return contextlib.nullcontext()


def quest_cpu(run, budget_s, threads=None):
    """The fp64 oracle (append + Quest selection + attention) on whole
    (sequence, KV head) units of successive decode steps at full context, as
    many as fit in budget_s, scaled to decode tokens/s of the whole batch."""
    from oracle import quest_decode_head
    cfg, x = run.cfg, run.x
    G, P = cfg.group, cfg.page_size
    units = [(b, h) for b in range(run.B) for h in range(cfg.num_kv_heads)]
    keys = {u: x["keys"][u[0], u[1]].cpu() for u in units}
    vals = {u: x["values"][u[0], u[1]].cpu() for u in units}
    q_h, kn_h, vn_h = x["q"].cpu(), x["k_new"].cpu(), x["v_new"].cpu()     # host copies, not timed
    done = 0
    with _limit_threads(threads) if threads else _limit_threads(None):
        t0 = time.perf_counter()
        for s in range(cfg.steps):
            for (b, h) in units:
                keys[(b, h)] = torch.cat([keys[(b, h)], kn_h[s, b, h][None]])
                vals[(b, h)] = torch.cat([vals[(b, h)], vn_h[s, b, h][None]])
                qs = q_h[s, b, h * G:(h + 1) * G]
                quest_decode_head(qs, keys[(b, h)], vals[(b, h)], P, cfg.top_k, W.default_scale(cfg.head_dim))
                done += 1
                if time.perf_counter() - t0 > budget_s:
                    break
            if time.perf_counter() - t0 > budget_s:
                break
        el = time.perf_counter() - t0
    tokens = done / cfg.num_kv_heads              # a token = one sequence's step over all its heads
    return dict(value=tokens / el, unit="tokens/s", cores=len(os.sched_getaffinity(0)), kind="oracle",
                threads=threads or _blas_threads(),
                sample=f"{done} (sequence, KV head) decode-step units of {cfg.name} at full context "
                       f"(append + Quest select + attention in fp64), {el:.1f} s",
                seconds=round(el, 2))


def h2o_cpu(run, budget_s):
    """The fp64 oracle's H2O decode step (append, attention with score
    accumulation, eviction) on (sequence, KV head) units of the compacted
    cache (state read from the GPU before timing, not timed), as many as fit
    in budget_s, scaled to decode tokens/s of the whole batch."""
    from oracle import H2OHeadState
    from oracle.h2o import h2o_step_head
    cfg, x = run.cfg, run.x
    G, D = cfg.group, cfg.head_dim
    L = int(run.kv.seq_lens[0])
    units = [(b, h) for b in range(run.B) for h in range(cfg.num_kv_heads)][:64]
    states = {}
    for (b, h) in units:
        k_, v_ = sp.read_slots(run.kv, b, h, L)
        states[(b, h)] = H2OHeadState.from_arrays(run.slot_pos[b, h, :L].cpu().numpy(), k_.cpu(), v_.cpu(),
                                                  run.scores[b, h, :L].double().cpu().numpy())
    q_h, kn_h, vn_h = x["q"].cpu(), x["k_new"].cpu(), x["v_new"].cpu()     # host copies, not timed
    done = 0
    t0 = time.perf_counter()
    for s in range(cfg.steps):
        for (b, h) in units:
            st = states[(b, h)]
            states[(b, h)] = h2o_step_head(st, q_h[s, b, h * G:(h + 1) * G], cfg.prompt + s, kn_h[s, b, h],
                                           vn_h[s, b, h], cfg.budget, cfg.recent_window, W.default_scale(D))[0]
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    return dict(value=done / cfg.num_kv_heads / el, unit="tokens/s", cores=len(os.sched_getaffinity(0)),
                kind="oracle", threads=_blas_threads(),
                sample=f"{done} (sequence, KV head) decode-step units of {cfg.name} (the first {len(units)} "
                       f"units, successive steps; append + attention + accumulate + evict in fp64), {el:.1f} s",
                seconds=round(el, 2))


def evicted_cpu(run, budget_s):
    """The fp64 oracle's dense decode over the retained slots (append, then
    attention of the group's query heads) on (sequence, KV head) units, as
    many as fit in budget_s, scaled to decode tokens/s of the whole batch."""
    from oracle import attend
    cfg, x = run.cfg, run.x
    G = cfg.group
    lens = x["lens"].tolist()
    units = [(b, h) for b in range(run.B) for h in range(cfg.num_kv_heads)]
    done, el = 0, 0.0
    for (b, h) in units:
        L = lens[b]
        # the unit's retained K/V and the new token, copied to host memory (not timed)
        kk = torch.cat([x["keys"][b, h, :L], x["k_new"][0, b, h][None]]).cpu()
        vv = torch.cat([x["values"][b, h, :L], x["v_new"][0, b, h][None]]).cpu()
        qh = x["q"][0, b, h * G:(h + 1) * G].cpu()
        t0 = time.perf_counter()
        kk64, vv64 = kk.double().numpy(), vv.double().numpy()
        for a in range(G):
            attend(qh[a].double().numpy(), kk64, vv64, W.default_scale(cfg.head_dim))
        el += time.perf_counter() - t0
        done += 1
        if el > budget_s:
            break
    return dict(value=done / cfg.num_kv_heads / el, unit="tokens/s", cores=len(os.sched_getaffinity(0)),
                kind="oracle", threads=_blas_threads(),
                sample=f"{done} (sequence, KV head) units of {cfg.name}'s first decode step (retained lengths "
                       f"512..2048, append + dense attention in fp64), {el:.1f} s", seconds=round(el, 2))


# oracle timings reported beside secondary workloads (bounded subsets)
CPU_SUBSETS = {
    "quest_gqa8_b4_ctx128k": lambda r, t: quest_cpu(r, t),
    "h2o_qwen3_8b_b32_prompt8k_bud1k": h2o_cpu,
    "evicted_b256_len512to2048": evicted_cpu,
}


def cpu_baseline(run, budget_s):
    """The headline's oracle timing at every core, with the same sample at one
    thread beside it."""
    full = quest_cpu(run, budget_s * 0.6)
    one = quest_cpu(run, budget_s * 0.4, threads=1)
    full["value_1_thread"] = one["value"]
    full["sample_1_thread"] = one["sample"]
    return full


def copy_calibration(dev):
    """A plain device copy of 1 GiB: reads 1 GiB, writes 1 GiB."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    ts = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4,
                      "copy_us": [round(t * 1e6, 1) for t in ts]}))


# ----------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--config", default=HEADLINE, choices=workload_names())
    ap.add_argument("--secondary", default="quest_llama3_8b_b16_ctx32k_two_launch,quest_f32_b1_h8_d64_ctx1k,"
                                           "quest_gqa8_b4_ctx128k,quest_gqa8_b4_ctx128k_two_launch,"
                                           "h2o_qwen3_8b_b32_prompt8k_bud1k,"
                                           "evicted_b256_len512to2048,"
                                           "quest_sink4_recent32_llama3_8b_b16_ctx32k,"
                                           "quest_groupmax_gqa8_b4_ctx128k,"
                                           "snapkv_qwen3_30b_a3b_b4_prompt128k_bud8k,"
                                           "h2o_prefill_qwen3_8b_b4_prompt32k_chunk8k_bud1k,"
                                           "omnikv_llama3_8b_b4_ctx128k_b4k",
                    help="comma-separated extra workloads reported under 'secondary' ('' for none)")
    ap.add_argument("--warm", action="store_true", help="skip the cache flush between steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU: every call of the library works on one device, "
              "so there is no multi-GPU run to measure", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = "cuda"
    if args.copy_calibration:
        copy_calibration(dev)
        return
    sp.load()
    spare = args.warmup + 2 * args.steps + 16

    run = make_run(args.config, dev, spare)
    per, step_t, wins, graph_t, ub, cb, wall = measure(run, args.steps, args.warmup, cold=not args.warm)
    res = summarize(run, per, step_t, wins, graph_t, ub, cb, args.config)

    secondary = {}
    for name in [n for n in args.secondary.split(",") if n and n != args.config]:
        r2 = make_run(name, dev, spare)
        p2, st2, w2, gt2, ub2, cb2, _ = measure(r2, args.steps, min(args.warmup, 2), cold=not args.warm)
        s2 = summarize(r2, p2, st2, w2, gt2, ub2, cb2, name)
        s2["config"] = r2.config()
        if not args.no_cpu_baseline and name in CPU_SUBSETS:
            s2["cpu_baseline"] = CPU_SUBSETS[name](r2, args.cpu_seconds / 4)
        secondary[name] = s2
        del r2
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline and isinstance(run, QuestRun):
        cpu = cpu_baseline(run, args.cpu_seconds)

    cfg = run.cfg
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
        "config": dict(run.config(), cache="cold (1 GiB flush before each step)" if not args.warm
                       else "warm", step="the step's calls launched back to back on one stream"),
        "graph_ms_per_step": res["graph_ms_per_step"],
        "windows": WINDOWS,
        "window_ms_per_step": res["window_ms_per_step"],
        "call_us": res["call_us"],
        "all_bytes_per_step": res["all_bytes_per_step"],
        "all_bytes_GBps": res["all_bytes_GBps"],
        "all_bytes_frac": res["all_bytes_frac"],
        "wall_s_timed_loop": wall,
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
