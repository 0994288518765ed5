"""Seeded input generators: deterministic, shaped as the named workloads, and
bookkeeping (block tables, lengths, positions) well-formed."""
import torch

import workloads as W


def test_config_names_and_seeds():
    assert len(W.CONFIGS) == 9
    seeds = [W.config_seed(n) for n in W.CONFIGS]
    assert seeds == list(range(1000, 1009))


def test_quest_inputs_deterministic_and_shaped():
    cfg = W.CONFIGS["quest_llama3_8b_b16_ctx32k"]
    a = W.quest_inputs(cfg, 7, context=100, batch=2)
    b = W.quest_inputs(cfg, 7, context=100, batch=2)
    assert a["keys"].shape == (2, 8, 100, 128) and a["keys"].dtype == torch.bfloat16
    assert a["q"].shape == (cfg.steps, 2, 32, 128)
    assert torch.equal(a["keys"], b["keys"]) and torch.equal(a["q"], b["q"])
    bt = a["block_table"]
    assert bt.shape == (2, a["max_pages"]) and bt.dtype == torch.int32
    assert len(set(bt.flatten().tolist())) == bt.numel()          # no block shared
    assert int(bt.max()) < a["num_blocks"]


def test_quest_outlier_channels():
    cfg = W.CONFIGS["quest_gqa8_b4_ctx128k"]
    x = W.quest_inputs(cfg, 3, context=512, batch=1)
    oc = x["outlier_channels"]
    assert oc.shape == (8, 3)
    k = x["keys"].float()
    for h in range(8):
        big = k[0, h, :, oc[h]].abs().mean()
        rest = k[0, h].abs().mean()
        assert big > 4 * rest


def test_h2o_inputs():
    cfg = W.CONFIGS["h2o_qwen3_8b_b32_prompt8k_bud1k"]
    x = W.h2o_inputs(cfg, 1, prompt=300, batch=2, steps=3)
    assert x["q_prompt"].shape == (2, 300, 32, 128) and x["q_prompt"].dtype == torch.bfloat16
    assert "prompt_scores" not in x
    # the stand-in scores are drawn only on request, after everything else
    y = W.h2o_inputs(cfg, 1, prompt=300, batch=2, steps=3, synthetic_prompt_scores=True)
    for k in ("keys", "values", "q_prompt", "q", "k_new", "v_new", "block_table"):
        assert torch.equal(x[k], y[k])
    s = y["prompt_scores"]
    assert s.shape == (2, 8, 300) and s.dtype == torch.float32 and bool((s > 0).all())
    # early tokens carry more stand-in mass on average
    assert s[..., :30].mean() > s[..., -30:].mean()


def test_evicted_inputs_positions_sorted_and_ragged():
    cfg = W.CONFIGS["evicted_b256_len512to2048"]
    x = W.evicted_inputs(cfg, 2, batch=3, min_len=5, max_len=40, steps=2)
    for b in range(3):
        L = int(x["lens"][b])
        assert 5 <= L <= 40
        for h in range(8):
            p = x["positions"][b, h, :L]
            assert bool((p[1:] > p[:-1]).all()) and int(p.max()) < x["source_len"]
            assert bool((x["positions"][b, h, L:] == -1).all())


def test_snapkv_inputs_shaped_and_salient():
    cfg = W.CONFIGS["snapkv_b2_h8_kv2_d128_prompt2k"]
    a = W.snapkv_inputs(cfg, 5, prompt=400, batch=2, steps=2)
    b = W.snapkv_inputs(cfg, 5, prompt=400, batch=2, steps=2)
    assert a["keys"].shape == (2, 2, 400, 128) and a["keys"].dtype == torch.bfloat16
    assert a["q_obs"].shape == (2, cfg.window, 8, 128)
    assert a["q"].shape == (2, 2, 8, 128)
    assert torch.equal(a["keys"], b["keys"]) and torch.equal(a["q_obs"], b["q_obs"])
    assert a["max_pages"] * cfg.page_size >= 402
    # the window queries lean toward the keys of position 0 (twice the gain)
    k0 = a["keys"][0, 0, 0].float()
    q = a["q_obs"][0, :, 0].float()
    assert float((q @ k0).mean()) > 3 * 128 ** 0.5


def test_h2o_prefill_inputs_shaped():
    cfg = W.CONFIGS["h2o_prefill_qwen3_8b_b4_prompt32k_chunk8k_bud1k"]
    a = W.h2o_prefill_inputs(cfg, 3, prompt=300, batch=2)
    b = W.h2o_prefill_inputs(cfg, 3, prompt=300, batch=2)
    assert a["keys"].shape == (2, 8, 300, 128) and a["q"].shape == (2, 300, 32, 128)
    assert torch.equal(a["q"], b["q"]) and torch.equal(a["keys"], b["keys"])
    assert a["max_pages"] * cfg.page_size >= cfg.budget + cfg.chunk


def test_omnikv_inputs_shaped():
    cfg = W.CONFIGS["omnikv_llama3_8b_b4_ctx128k_b4k"]
    a = W.omnikv_inputs(cfg, 4, context=200, batch=2)
    assert a["keys_obs"].shape == a["keys"].shape == (2, 8, 200, 128)
    assert a["q_obs"].shape == (cfg.steps, 2, 32, 128)
    assert not torch.equal(a["keys_obs"], a["keys"])
    assert a["block_table"].shape == (2, a["max_pages"])
