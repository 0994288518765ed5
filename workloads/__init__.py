"""Seeded synthetic inputs for sparse decode attention (Quest selection, H2O eviction).

This module only draws random tensors and lays out bookkeeping (lengths, block
tables, slot positions).  It holds none of the method's arithmetic: no page
extrema, no bounds, no softmax, no selection.  Both the CPU oracle and the HIP
path receive the same tensors from here.

The shapes follow the long-context agent decode workloads of
"SparseEngine: Sparse-First Inference Engine" (Appendix C.6 "Overall Serving
Performance": 131,072-token inputs; Appendix C.7: 32,768-token inputs) scaled
to one attention layer of Llama-3-8B / Qwen3-8B-shaped models.  No dataset or
model weights are used: keys, values and queries are Gaussian draws.

Every draw comes from one ``torch.Generator`` seeded by the caller, in a fixed
order (scales, keys, values, prompt queries, per-step queries, per-step new
keys/values, block permutation; anything drawn only on request comes last), on
the device the caller names.  bf16 tensors
are drawn in fp32 and rounded to nearest-even by ``Tensor.to``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

__all__ = [
    "QuestConfig", "H2OConfig", "EvictedConfig", "SnapKVConfig", "H2OPrefillConfig", "CONFIGS",
    "config_seed", "quest_inputs", "h2o_inputs", "evicted_inputs", "snapkv_inputs",
    "h2o_prefill_inputs", "OmniKVConfig", "omnikv_inputs", "random_block_table",
    "torch_dtype",
]


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


@dataclasses.dataclass(frozen=True)
class QuestConfig:
    """Quest decode: every token stays resident, pages are selected per KV head."""
    name: str
    dtype: str            # "f32" | "bf16"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    context: int          # tokens resident before the first decode step
    page_size: int
    top_k: int            # pages read per KV head
    steps: int            # decode steps (each appends one token)
    kv_channel_scale_sigma: float = 0.0   # >0: per-(kv-head, channel) LogNormal(0, sigma) scale
    key_outlier_frac: float = 0.0         # fraction of key channels per KV head that are outliers
    key_outlier_mag: float = 1.0          # multiplier applied to outlier key channels

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_pages(self) -> int:
        return -(-(self.context + self.steps) // self.page_size)


@dataclasses.dataclass(frozen=True)
class H2OConfig:
    """H2O online eviction: the prompt is compacted to ``budget`` slots, then
    every decode step appends one token, accumulates probabilities and evicts."""
    name: str
    dtype: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    prompt: int
    budget: int
    recent_window: int
    steps: int
    page_size: int = 16

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def slot_cap(self) -> int:
        # slots needed: the whole prompt before its compaction, or budget + 1
        return max(self.prompt, self.budget + 1)

    @property
    def max_pages(self) -> int:
        return -(-self.slot_cap // self.page_size)


@dataclasses.dataclass(frozen=True)
class EvictedConfig:
    """Dense decode over physically retained (already evicted) KV with ragged
    per-sequence slot counts; each step appends one token, nothing is evicted."""
    name: str
    dtype: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    min_len: int
    max_len: int
    source_len: int       # logical positions are a sorted sample of [0, source_len)
    steps: int
    page_size: int = 16

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_pages(self) -> int:
        return -(-(self.max_len + self.steps) // self.page_size)


@dataclasses.dataclass(frozen=True)
class SnapKVConfig:
    """SnapKV prompt selection: the window queries score the earlier prompt
    positions, the pooled scores pick ``budget - window`` of them, the cache
    is compacted, then decoding runs over the retained slots.

    Keys carry a shared per-(sequence, KV head) direction on a sparse set of
    runs of positions ("salient" runs, plus position 0 at twice the gain) that
    the window queries also carry, so that attention concentrates on them the
    way it does on important prompt spans; everything else is Gaussian."""
    name: str
    dtype: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    prompt: int
    window: int
    pool_kernel: int
    budget: int
    n_sink: int
    steps: int
    page_size: int = 16
    salient_frac: float = 0.03     # fraction of positions inside salient runs
    salient_run: int = 8           # positions per run
    key_gain: float = 8.0          # salient keys: + key_gain * direction
    query_gain: float = 0.5        # window queries: + query_gain * sqrt(D) * direction

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_pages(self) -> int:
        return -(-(self.prompt + self.steps) // self.page_size)


@dataclasses.dataclass(frozen=True)
class H2OPrefillConfig:
    """H2O over a prompt prefilled chunk by chunk: each chunk is appended, its
    queries' attention probabilities are added to the scores of every
    available slot, and the cache is evicted to the budget.  Keys and
    queries share a per-(sequence, KV head) direction on a sparse set of keys
    (as for SnapKV) so that attention concentrates."""
    name: str
    dtype: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    prompt: int
    chunk: int
    budget: int
    recent_window: int
    page_size: int = 16
    hot_frac: float = 0.05        # keys carrying the shared direction
    key_gain: float = 6.0
    query_gain: float = 0.5       # queries: + query_gain * sqrt(D) * direction

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_pages(self) -> int:
        return -(-(self.budget + self.chunk) // self.page_size)


@dataclasses.dataclass(frozen=True)
class OmniKVConfig:
    """OmniKV decode: an observation layer selects top_b token positions from
    its current queries; a sparse layer with its own cache attends over them.
    Keys of both layers carry a per-(sequence, KV head) direction on a sparse
    set of positions shared by the layers (important spans persist across
    nearby layers), which the queries also carry."""
    name: str
    dtype: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    context: int
    top_b: int
    steps: int
    page_size: int = 16
    hot_frac: float = 0.02
    key_gain: float = 6.0
    query_gain: float = 0.5

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_pages(self) -> int:
        return -(-self.context // self.page_size)


CONFIGS = {
    # Quest sparse decode, one layer, fp32, parity-sized.
    "quest_f32_b1_h8_d64_ctx1k": QuestConfig(
        "quest_f32_b1_h8_d64_ctx1k", "f32", batch=1, num_q_heads=8, num_kv_heads=8,
        head_dim=64, context=1024, page_size=16, top_k=8, steps=1),
    # Quest sparse decode, Llama-3-8B-shaped attention layer.
    "quest_llama3_8b_b16_ctx32k": QuestConfig(
        "quest_llama3_8b_b16_ctx32k", "bf16", batch=16, num_q_heads=32, num_kv_heads=8,
        head_dim=128, context=32768, page_size=16, top_k=128, steps=32,
        kv_channel_scale_sigma=0.5),
    # H2O online eviction, Qwen3-8B-shaped attention layer.
    "h2o_qwen3_8b_b32_prompt8k_bud1k": H2OConfig(
        "h2o_qwen3_8b_b32_prompt8k_bud1k", "bf16", batch=32, num_q_heads=32, num_kv_heads=8,
        head_dim=128, prompt=8192, budget=1024, recent_window=128, steps=256),
    # Large-batch decode over physically evicted KV.
    "evicted_b256_len512to2048": EvictedConfig(
        "evicted_b256_len512to2048", "bf16", batch=256, num_q_heads=32, num_kv_heads=8,
        head_dim=128, min_len=512, max_len=2048, source_len=8192, steps=64),
    # Long-context Quest decode, GQA 8, keys with outlier channels.
    "quest_gqa8_b4_ctx128k": QuestConfig(
        "quest_gqa8_b4_ctx128k", "bf16", batch=4, num_q_heads=64, num_kv_heads=8,
        head_dim=128, context=131072, page_size=32, top_k=128, steps=16,
        key_outlier_frac=0.02, key_outlier_mag=8.0),
    # SnapKV prompt selection, parity-sized.
    "snapkv_b2_h8_kv2_d128_prompt2k": SnapKVConfig(
        "snapkv_b2_h8_kv2_d128_prompt2k", "bf16", batch=2, num_q_heads=8, num_kv_heads=2,
        head_dim=128, prompt=2048, window=32, pool_kernel=7, budget=512, n_sink=0, steps=4),
    # SnapKV prompt selection over 131,072-token prompts, Qwen3-30B-A3B-shaped
    # attention layer (32 query heads, 4 KV heads), 8,192-token budget.
    "snapkv_qwen3_30b_a3b_b4_prompt128k_bud8k": SnapKVConfig(
        "snapkv_qwen3_30b_a3b_b4_prompt128k_bud8k", "bf16", batch=4, num_q_heads=32,
        num_kv_heads=4, head_dim=128, prompt=131072, window=32, pool_kernel=7, budget=8192,
        n_sink=0, steps=16),
    # H2O chunk-wise prefill of 32,768-token prompts in 8,192-token chunks,
    # Qwen3-8B-shaped attention layer, budget 1024 with a 128-token window.
    "h2o_prefill_qwen3_8b_b4_prompt32k_chunk8k_bud1k": H2OPrefillConfig(
        "h2o_prefill_qwen3_8b_b4_prompt32k_chunk8k_bud1k", "bf16", batch=4, num_q_heads=32,
        num_kv_heads=8, head_dim=128, prompt=32768, chunk=8192, budget=1024, recent_window=128),
    # OmniKV decode over 131,072-token contexts, Llama-3-8B-shaped layers,
    # 4,096 selected tokens reused by the sparse layer.
    "omnikv_llama3_8b_b4_ctx128k_b4k": OmniKVConfig(
        "omnikv_llama3_8b_b4_ctx128k_b4k", "bf16", batch=4, num_q_heads=32, num_kv_heads=8,
        head_dim=128, context=131072, top_b=4096, steps=8),
}

_CONFIG_ORDER = list(CONFIGS)


def config_seed(name: str) -> int:
    """Seed of a named workload: 1000 + its index in CONFIGS."""
    return 1000 + _CONFIG_ORDER.index(name)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(g, shape, device, dtype=torch.float32):
    return torch.randn(*shape, generator=g, device=device, dtype=dtype)


def random_block_table(batch: int, max_pages: int, g: torch.Generator, device,
                       num_blocks: Optional[int] = None) -> tuple[torch.Tensor, int]:
    """Block table [batch][max_pages] int32: a seeded random permutation of the
    physical blocks, so that no sequence's pages are contiguous by luck."""
    n = batch * max_pages if num_blocks is None else num_blocks
    perm = torch.randperm(n, generator=g, device=device).to(torch.int32)
    return perm[: batch * max_pages].reshape(batch, max_pages).contiguous(), n


def quest_inputs(cfg: QuestConfig, seed: int, device="cpu", context: Optional[int] = None,
                 batch: Optional[int] = None, spare_tokens: int = 0) -> dict:
    """Logical keys/values [B][H_kv][L0][D] resident before decoding, per-step
    queries [S][B][H_q][D] and per-step new keys/values [S][B][H_kv][D], plus a
    scattered block table.  ``context``/``batch`` override the config's sizes
    (for reduced parity cases); ``spare_tokens`` adds cache capacity beyond the
    config's steps (for runs that decode more steps than the config)."""
    L0 = cfg.context if context is None else context
    B = cfg.batch if batch is None else batch
    H, Hq, D, S = cfg.num_kv_heads, cfg.num_q_heads, cfg.head_dim, cfg.steps
    dt = torch_dtype(cfg.dtype)
    g = _gen(seed, device)
    # scales first (drawn even when unused so that the draw order is fixed)
    sk = torch.exp(cfg.kv_channel_scale_sigma * _randn(g, (H, D), device))
    sv = torch.exp(cfg.kv_channel_scale_sigma * _randn(g, (H, D), device))
    n_out = int(round(cfg.key_outlier_frac * D))
    out_ch = torch.stack([torch.randperm(D, generator=g, device=device)[:n_out] for _ in range(H)]) \
        if n_out > 0 else torch.zeros((H, 0), dtype=torch.long, device=device)
    kmul = torch.ones(H, D, device=device)
    for h in range(H):
        kmul[h, out_ch[h]] = cfg.key_outlier_mag
    kscale = (sk * kmul)[None, :, None, :]
    vscale = sv[None, :, None, :]
    keys = (_randn(g, (B, H, L0, D), device) * kscale).to(dt)
    values = (_randn(g, (B, H, L0, D), device) * vscale).to(dt)
    q = _randn(g, (S, B, Hq, D), device).to(dt)
    k_new = (_randn(g, (S, B, H, D), device) * kscale[:, :, 0, :]).to(dt)
    v_new = (_randn(g, (S, B, H, D), device) * vscale[:, :, 0, :]).to(dt)
    max_pages = -(-(L0 + S + spare_tokens) // cfg.page_size)
    bt, nblk = random_block_table(B, max_pages, g, device)
    return dict(keys=keys, values=values, q=q, k_new=k_new, v_new=v_new,
                block_table=bt, num_blocks=nblk, max_pages=max_pages,
                context=L0, batch=B, outlier_channels=out_ch)


def harmonic(n: torch.Tensor) -> torch.Tensor:
    """H_n = sum_{i<=n} 1/i for integer tensors n >= 0 (H_0 = 0)."""
    m = int(n.max().item()) if n.numel() else 0
    h = torch.cat([torch.zeros(1, dtype=torch.float64),
                   torch.cumsum(1.0 / torch.arange(1, m + 1, dtype=torch.float64), 0)])
    return h[n.cpu().long()].to(n.device)


def h2o_inputs(cfg: H2OConfig, seed: int, device="cpu", prompt: Optional[int] = None,
               batch: Optional[int] = None, steps: Optional[int] = None,
               synthetic_prompt_scores: bool = False) -> dict:
    """Prompt keys/values [B][H_kv][n][D], the prompt's queries [B][n][H_q][D],
    per-step queries / new keys / new values, and a block table.

    The prompt's H2O scores are not input data: they are the attention
    probabilities its own queries give during prefill (the whole prompt is one
    prefill chunk of n <= 8192 tokens, causal), which sp_h2o_prefill_scores
    computes on the GPU and oracle.h2o_prefill_chunk on the CPU; the initial
    compaction to the budget then evicts on them.

    synthetic_prompt_scores: also return a seeded stand-in [B][H_kv][n] (fp32),
    drawn after everything else so the other tensors do not change, for tests
    that only need some score state: G * (H_n - H_{j-1}) (the mass token j, 1-based,
    collects under uniform causal attention) times LogNormal(0, 1)."""
    n = cfg.prompt if prompt is None else prompt
    B = cfg.batch if batch is None else batch
    S = cfg.steps if steps is None else steps
    H, Hq, D, G = cfg.num_kv_heads, cfg.num_q_heads, cfg.head_dim, cfg.group
    dt = torch_dtype(cfg.dtype)
    g = _gen(seed, device)
    keys = _randn(g, (B, H, n, D), device).to(dt)
    values = _randn(g, (B, H, n, D), device).to(dt)
    q_prompt = _randn(g, (B, n, Hq, D), device).to(dt)
    q = _randn(g, (S, B, Hq, D), device).to(dt)
    k_new = _randn(g, (S, B, H, D), device).to(dt)
    v_new = _randn(g, (S, B, H, D), device).to(dt)
    max_pages = -(-max(n, cfg.budget + 1) // cfg.page_size)
    bt, nblk = random_block_table(B, max_pages, g, device)
    out = dict(keys=keys, values=values, q_prompt=q_prompt, q=q, k_new=k_new, v_new=v_new, block_table=bt,
               num_blocks=nblk, max_pages=max_pages, prompt=n, batch=B, steps=S)
    if synthetic_prompt_scores:
        j = torch.arange(1, n + 1)
        base = (G * (harmonic(torch.full_like(j, n)) - harmonic(j - 1))).to(torch.float32).to(device)
        skew = torch.exp(_randn(g, (B, H, n), device))
        out["prompt_scores"] = (base[None, None, :] * skew).to(torch.float32)
    return out


def evicted_inputs(cfg: EvictedConfig, seed: int, device="cpu", batch: Optional[int] = None,
                   min_len: Optional[int] = None, max_len: Optional[int] = None,
                   steps: Optional[int] = None) -> dict:
    """Retained KV after a physical eviction: per-sequence slot counts
    L_b ~ U{min_len..max_len}, per-(sequence, head) retained logical positions
    (a sorted sample of [0, source_len)), keys/values [B][H_kv][max_len][D]
    (entries at slots >= L_b are padding), per-step queries and new tokens."""
    B = cfg.batch if batch is None else batch
    lo = cfg.min_len if min_len is None else min_len
    hi = cfg.max_len if max_len is None else max_len
    S = cfg.steps if steps is None else steps
    H, Hq, D = cfg.num_kv_heads, cfg.num_q_heads, cfg.head_dim
    dt = torch_dtype(cfg.dtype)
    g = _gen(seed, device)
    lens = torch.randint(lo, hi + 1, (B,), generator=g, device=device, dtype=torch.int32)
    keys = _randn(g, (B, H, hi, D), device).to(dt)
    values = _randn(g, (B, H, hi, D), device).to(dt)
    src = max(cfg.source_len, hi)
    pos = torch.full((B, H, hi), -1, dtype=torch.int32, device=device)
    for b in range(B):
        L = int(lens[b])
        for h in range(H):
            pick = torch.randperm(src, generator=g, device=device)[:L]
            pos[b, h, :L] = torch.sort(pick).values.to(torch.int32)
    q = _randn(g, (S, B, Hq, D), device).to(dt)
    k_new = _randn(g, (S, B, H, D), device).to(dt)
    v_new = _randn(g, (S, B, H, D), device).to(dt)
    max_pages = -(-(hi + S) // cfg.page_size)
    bt, nblk = random_block_table(B, max_pages, g, device)
    return dict(keys=keys, values=values, lens=lens, positions=pos, q=q, k_new=k_new,
                v_new=v_new, block_table=bt, num_blocks=nblk, max_pages=max_pages,
                batch=B, source_len=src, steps=S)


def default_scale(head_dim: int) -> float:
    """Softmax temperature 1/sqrt(d_k) used by every workload."""
    return 1.0 / math.sqrt(head_dim)


def snapkv_inputs(cfg: SnapKVConfig, seed: int, device="cpu", prompt: Optional[int] = None,
                  batch: Optional[int] = None, steps: Optional[int] = None) -> dict:
    """Prompt keys/values [B][H_kv][n][D], window queries [B][w][H_q][D] (the
    queries of positions n - w .. n - 1), per-step decode queries / new keys /
    new values, and a scattered block table.

    Draw order: directions [B][H_kv][D] (normalised), salient-run starts,
    key noise, values, window-query noise, decode queries, new keys, new
    values, block permutation."""
    n = cfg.prompt if prompt is None else prompt
    B = cfg.batch if batch is None else batch
    S = cfg.steps if steps is None else steps
    H, Hq, D, G, w = cfg.num_kv_heads, cfg.num_q_heads, cfg.head_dim, cfg.group, cfg.window
    dt = torch_dtype(cfg.dtype)
    g = _gen(seed, device)
    dirs = _randn(g, (B, H, D), device)
    dirs = dirs / dirs.norm(dim=-1, keepdim=True)
    n_runs = max(1, int(round(cfg.salient_frac * n / cfg.salient_run)))
    starts = torch.randint(0, max(1, n - cfg.salient_run), (B, H, n_runs), generator=g, device=device)
    gain = torch.zeros(B, H, n, device=device)
    offs = torch.arange(cfg.salient_run, device=device)
    idx = (starts[..., None] + offs).clamp(max=n - 1).reshape(B, H, -1)
    gain.scatter_(2, idx, 1.0)
    gain[:, :, 0] = 2.0
    keys = (_randn(g, (B, H, n, D), device) + cfg.key_gain * gain[..., None] * dirs[:, :, None, :]).to(dt)
    values = _randn(g, (B, H, n, D), device).to(dt)
    qdir = dirs.repeat_interleave(G, dim=1)                                  # [B][Hq][D]
    q_obs = (_randn(g, (B, w, Hq, D), device) +
             cfg.query_gain * math.sqrt(D) * qdir[:, None, :, :]).to(dt)
    q = _randn(g, (S, B, Hq, D), device).to(dt)
    k_new = _randn(g, (S, B, H, D), device).to(dt)
    v_new = _randn(g, (S, B, H, D), device).to(dt)
    max_pages = -(-(n + S) // cfg.page_size)
    bt, nblk = random_block_table(B, max_pages, g, device)
    return dict(keys=keys, values=values, q_obs=q_obs, q=q, k_new=k_new, v_new=v_new,
                block_table=bt, num_blocks=nblk, max_pages=max_pages, prompt=n, batch=B, steps=S)


def h2o_prefill_inputs(cfg: H2OPrefillConfig, seed: int, device="cpu", prompt: Optional[int] = None,
                       batch: Optional[int] = None) -> dict:
    """Prompt keys/values [B][H_kv][n][D], queries [B][n][H_q][D], a block
    table for budget + chunk slots.  Draw order: directions, hot-key mask,
    key noise, values, query noise, block permutation."""
    n = cfg.prompt if prompt is None else prompt
    B = cfg.batch if batch is None else batch
    H, Hq, D, G = cfg.num_kv_heads, cfg.num_q_heads, cfg.head_dim, cfg.group
    dt = torch_dtype(cfg.dtype)
    g = _gen(seed, device)
    dirs = _randn(g, (B, H, D), device)
    dirs = dirs / dirs.norm(dim=-1, keepdim=True)
    hot = (torch.rand(B, H, n, generator=g, device=device) < cfg.hot_frac).to(torch.float32)
    keys = (_randn(g, (B, H, n, D), device) + cfg.key_gain * hot[..., None] * dirs[:, :, None, :]).to(dt)
    values = _randn(g, (B, H, n, D), device).to(dt)
    q = (_randn(g, (B, n, Hq, D), device)
         + cfg.query_gain * math.sqrt(D) * dirs.repeat_interleave(G, dim=1)[:, None]).to(dt)
    max_pages = cfg.max_pages
    bt, nblk = random_block_table(B, max_pages, g, device)
    return dict(keys=keys, values=values, q=q, block_table=bt, num_blocks=nblk, max_pages=max_pages,
                prompt=n, batch=B)


def omnikv_inputs(cfg: OmniKVConfig, seed: int, device="cpu", context: Optional[int] = None,
                  batch: Optional[int] = None) -> dict:
    """Two layers (observation, sparse) of keys/values [B][H_kv][L][D],
    per-step queries of both layers [S][B][H_q][D], one block table (the
    layers share the paging).  Draw order: directions, hot mask, then per
    layer keys and values, then per layer queries, block permutation."""
    L = cfg.context if context is None else context
    B = cfg.batch if batch is None else batch
    H, Hq, D, G, S = cfg.num_kv_heads, cfg.num_q_heads, cfg.head_dim, cfg.group, cfg.steps
    dt = torch_dtype(cfg.dtype)
    g = _gen(seed, device)
    dirs = _randn(g, (B, H, D), device)
    dirs = dirs / dirs.norm(dim=-1, keepdim=True)
    hot = (torch.rand(B, H, L, generator=g, device=device) < cfg.hot_frac).to(torch.float32)
    layers = []
    for _ in range(2):
        k = (_randn(g, (B, H, L, D), device) + cfg.key_gain * hot[..., None] * dirs[:, :, None, :]).to(dt)
        v = _randn(g, (B, H, L, D), device).to(dt)
        layers.append((k, v))
    qs = []
    for _ in range(2):
        qs.append((_randn(g, (S, B, Hq, D), device)
                   + cfg.query_gain * math.sqrt(D) * dirs.repeat_interleave(G, dim=1)[None]).to(dt))
    bt, nblk = random_block_table(B, cfg.max_pages if context is None else -(-L // cfg.page_size), g, device)
    return dict(keys_obs=layers[0][0], values_obs=layers[0][1], keys=layers[1][0], values=layers[1][1],
                q_obs=qs[0], q=qs[1], block_table=bt, num_blocks=nblk, context=L, batch=B,
                max_pages=-(-L // cfg.page_size))
