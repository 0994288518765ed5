"""Pins for oracle.quest: brute force, closed forms, invariants, the pages'
eight-token example, and torch SDPA for the all-pages special case."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import (page_extrema, page_bound, group_bound, select_top_pages,
                    quest_decode_head, quest_decode)
from oracle.quest import forced_pages

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_values(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16).to(torch.float64).numpy()


# ---------------------------------------------------------------- extrema
@pytest.mark.parametrize("L,P", [(1, 16), (16, 16), (37, 16), (64, 32), (9, 1)])
def test_page_extrema_brute_force(L, P):
    keys = _bf16_values((L, 5), seed=L * 7 + P)
    mins, maxs = page_extrema(keys, P)
    assert mins.shape == (-(-L // P), 5)
    for p in range(mins.shape[0]):
        for c in range(5):
            lo, hi = math.inf, -math.inf
            for t in range(p * P, min(L, (p + 1) * P)):   # plain scan, valid tokens only
                lo = keys[t, c] if keys[t, c] < lo else lo
                hi = keys[t, c] if keys[t, c] > hi else hi
            assert mins[p, c] == lo and maxs[p, c] == hi


# ---------------------------------------------------------------- bound
@pytest.mark.parametrize("P", [2, 16, 32])
def test_bound_upper_bounds_every_token_logit(P):
    D, L = 64, 40 * P + 5
    keys = _bf16_values((L, D), seed=P, scale=2.0)
    q = _bf16_values((D,), seed=P + 100)
    mins, maxs = page_extrema(keys, P)
    U = page_bound(q, mins, maxs)
    for p in range(len(U)):
        tok = keys[p * P: min(L, (p + 1) * P)]
        logits = tok @ q
        slack = 1e-12 * float(np.abs(q) @ np.abs(tok).max(axis=0))
        assert U[p] >= logits.max() - slack
    # and it is not simply the max logit: for pages of >1 token it is strictly
    # larger somewhere (channels reach their extrema at different tokens)
    assert any(U[p] > (keys[p * P:(p + 1) * P] @ q).max() + 1e-9 for p in range(len(U) - 1))


def test_bound_page_size_one_is_the_exact_logit():
    keys = _bf16_values((50, 32), seed=3)
    q = _bf16_values((32,), seed=4)
    mins, maxs = page_extrema(keys, 1)
    U = page_bound(q, mins, maxs)
    for t in range(50):
        exact = sum(float(q[c]) * float(keys[t, c]) for c in range(32))
        assert abs(U[t] - exact) < 1e-12


def test_bound_nonnegative_query_is_dot_with_max():
    keys = _bf16_values((48, 16), seed=11)
    q = np.abs(_bf16_values((16,), seed=12))
    mins, maxs = page_extrema(keys, 16)
    np.testing.assert_allclose(page_bound(q, mins, maxs), maxs @ q, atol=1e-12)
    # and a non-positive query pairs with the minimum
    np.testing.assert_allclose(page_bound(-q, mins, maxs), mins @ (-q), atol=1e-12)


def test_bound_is_tight_when_one_token_holds_the_useful_extrema():
    q = np.array([1.0, -2.0, 0.5, -0.25])
    best = np.array([3.0, -4.0, 2.0, -1.0])          # max where q>0, min where q<0
    others = np.array([[1.0, 0.0, 1.5, 0.0], [-2.0, -3.0, 0.0, 0.5]])
    keys = np.vstack([others, best[None, :]])
    mins, maxs = page_extrema(keys, 3)
    assert page_bound(q, mins, maxs)[0] == pytest.approx(float(best @ q), abs=0)


def test_group_bound_sums_query_heads():
    keys = _bf16_values((64, 8), seed=21)
    qs = _bf16_values((4, 8), seed=22)
    mins, maxs = page_extrema(keys, 16)
    per_head = [[max(qs[a, c] * mins[p, c], qs[a, c] * maxs[p, c]) for c in range(8)]
                for a in range(4) for p in range(4)]
    expect = [sum(sum(per_head[a * 4 + p]) for a in range(4)) for p in range(4)]
    np.testing.assert_allclose(group_bound(qs, mins, maxs), expect, atol=1e-12)


# ---------------------------------------------------------------- top-k
def _brute_force_top(scores, k):
    """Enumerate every subset of size min(k, n); keep the one whose
    descending list of (score, -index) is lexicographically largest."""
    n = len(scores)
    best = None
    for sub in itertools.combinations(range(n), min(k, n)):
        key = sorted(((scores[p], -p) for p in sub), reverse=True)
        if best is None or key > best[0]:
            best = (key, sub)
    return sorted(best[1])


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(-3, 3), min_size=1, max_size=7), st.integers(1, 8))
def test_select_top_pages_brute_force_with_ties(vals, k):
    scores = [float(v) for v in vals]        # small integers force many ties
    assert select_top_pages(scores, k) == _brute_force_top(scores, k)


@settings(max_examples=100, deadline=None)
@given(st.lists(st.floats(-1e6, 1e6, allow_nan=False), min_size=1, max_size=300),
       st.integers(1, 64))
def test_select_top_pages_properties(scores, k):
    sel = select_top_pages(scores, k)
    assert len(sel) == min(k, len(scores))
    assert sel == sorted(set(sel))
    chosen = set(sel)
    for p in range(len(scores)):
        if p in chosen:
            continue
        for s in sel:      # every unselected page ranks below every selected one
            assert scores[p] < scores[s] or (scores[p] == scores[s] and p > s)


# ---------------------------------------------------------------- variants
# Section 5 of the pages: a Quest baseline with 4 sink pages, 32 recent pages
# and 92 selected pages; and the max-over-group aggregation of the bound.
@pytest.mark.parametrize("n,s,r", [(10, 2, 3), (4, 4, 32), (200, 4, 32), (3, 0, 0), (1, 1, 1)])
def test_forced_pages_enumerated(n, s, r):
    expect = [p for p in range(n) if p < s or p >= n - r]
    assert forced_pages(n, s, r) == expect


def _brute_force_forced(scores, k, forced):
    """Every subset of size min(k, n) that contains the forced pages; keep the
    one whose other members, as a descending list of (score, -index), are
    lexicographically largest."""
    n = len(scores)
    fs = set(forced)
    best = None
    for sub in itertools.combinations(range(n), min(k, n)):
        if not fs <= set(sub):
            continue
        key = sorted(((scores[p], -p) for p in sub if p not in fs), reverse=True)
        if best is None or key > best[0]:
            best = (key, sub)
    return sorted(best[1])


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(-3, 3), min_size=1, max_size=8), st.integers(1, 8),
       st.integers(0, 3), st.integers(0, 3))
def test_select_with_forced_pages_brute_force(vals, k, n_sink, n_recent):
    if n_sink + n_recent > k:
        return
    scores = [float(v) for v in vals]
    forced = forced_pages(len(scores), n_sink, n_recent)
    sel = select_top_pages(scores, k, forced)
    assert sel == _brute_force_forced(scores, k, forced)
    assert set(forced) <= set(sel)


def test_vortex_budget_4_sink_32_recent_92_selected():
    rng = np.random.default_rng(5)
    scores = rng.standard_normal(200)
    sel = select_top_pages(scores, 128, forced_pages(200, 4, 32))
    assert len(sel) == 128
    assert sel[:4] == [0, 1, 2, 3] and sel[-32:] == list(range(168, 200))
    middle = sel[4:-32]
    rest = list(range(4, 168))
    assert middle == sorted(sorted(rest, key=lambda p: -scores[p])[:92])


def test_no_forced_pages_is_plain_top_k():
    rng = np.random.default_rng(6)
    scores = rng.standard_normal(12)
    assert select_top_pages(scores, 5, forced_pages(12, 0, 0)) == _brute_force_top(list(scores), 5)


def test_group_max_with_one_head_equals_sum():
    keys = _bf16_values((64, 8), seed=31)
    qs = _bf16_values((1, 8), seed=32)
    mins, maxs = page_extrema(keys, 16)
    np.testing.assert_array_equal(group_bound(qs, mins, maxs, "max"), group_bound(qs, mins, maxs, "sum"))


def test_group_max_is_the_largest_head_bound():
    keys = _bf16_values((64, 8), seed=41)
    qs = _bf16_values((4, 8), seed=42)
    mins, maxs = page_extrema(keys, 16)
    expect = [max(sum(max(qs[a, c] * mins[p, c], qs[a, c] * maxs[p, c]) for c in range(8))
                  for a in range(4)) for p in range(4)]
    np.testing.assert_allclose(group_bound(qs, mins, maxs, "max"), expect, atol=1e-12)


def test_group_max_page_size_one_is_the_largest_head_logit():
    keys = _bf16_values((20, 16), seed=51)
    qs = _bf16_values((8, 16), seed=52)
    mins, maxs = page_extrema(keys, 1)
    S = group_bound(qs, mins, maxs, "max")
    for t in range(20):
        exact = max(sum(float(qs[a, c]) * float(keys[t, c]) for c in range(16)) for a in range(8))
        assert abs(S[t] - exact) < 1e-12


def test_quest_head_with_only_forced_pages_attends_exactly_them():
    P, L = 16, 16 * 20 + 5
    keys = _bf16_values((L, 32), seed=61)
    vals = _bf16_values((L, 32), seed=62)
    qs = _bf16_values((2, 32), seed=63)
    r = quest_decode_head(qs, keys, vals, P, 6, 0.2, n_sink=2, n_recent=4)
    assert r["selected"] == [0, 1, 17, 18, 19, 20]
    expect_tokens = np.concatenate([np.arange(0, 32), np.arange(17 * 16, L)])
    np.testing.assert_array_equal(r["tokens"], expect_tokens)


# ---------------------------------------------------------------- worked example
def test_quest_eight_token_example():
    """Eight tokens in four two-token pages, two pages loaded.  Values are
    chosen so every bound is computable by hand (q = [1, -1], D = 2):
      page 0: k0=[1,0],   k1=[0,1]    m=[0,0],    M=[1,1]  U = 1 + 0 = 1
      page 1: k2=[2,2],   k3=[-1,-3]  m=[-1,-3],  M=[2,2]  U = 2 + 3 = 5
      page 2: k4=[3,3],   k5=[0,0]    m=[0,0],    M=[3,3]  U = 3 + 0 = 3
      page 3: k6=[.5,-1], k7=[1,2]    m=[.5,-1],  M=[1,2]  U = 1 + 1 = 2
    Top-2 by the bound = pages {1, 2}.  (By the true maximum logit per page,
    1, 2, 0, 1.5, it would be {1, 3}: the bound is not the max logit.)
    Attention with scale 1 reads tokens 2..5, logits [0, 2, 0, 0]; with
    v_t = [t, 1]: o = [(2 + 3e^2 + 4 + 5)/(3 + e^2), 1], lse = log(3 + e^2)."""
    with open(os.path.join(GOLDEN, "quest_eight_token_history.json")) as f:
        ex = json.load(f)
    keys = np.array([[1, 0], [0, 1], [2, 2], [-1, -3], [3, 3], [0, 0], [.5, -1], [1, 2]],
                    dtype=np.float64)
    assert keys.shape[0] == ex["history_tokens"]
    values = np.array([[t, 1.0] for t in range(8)])
    q = np.array([[1.0, -1.0]])
    r = quest_decode_head(q, keys, values, ex["page_size"], ex["pages_loaded"], 1.0)
    assert len(r["scores"]) == ex["num_pages"]
    np.testing.assert_array_equal(r["scores"], [1, 5, 3, 2])
    assert r["selected"] == [1, 2]
    np.testing.assert_array_equal(r["tokens"], [2, 3, 4, 5])
    e2 = math.exp(2)
    np.testing.assert_allclose(r["out"][0], [(11 + 3 * e2) / (3 + e2), 1.0], atol=1e-14)
    assert r["lse"][0] == pytest.approx(math.log(3 + e2), abs=1e-14)


# ---------------------------------------------------------------- full step
@pytest.mark.parametrize("G,P,L", [(1, 16, 100), (4, 16, 257), (8, 32, 200)])
def test_all_pages_selected_equals_dense_sdpa(G, P, L):
    D = 64
    q = _bf16_values((G, D), seed=G + P)
    keys = _bf16_values((L, D), seed=L)
    values = _bf16_values((L, D), seed=L + 1)
    n_pages = -(-L // P)
    r = quest_decode_head(q, keys, values, P, n_pages + 3, 1 / math.sqrt(D))
    assert r["selected"] == list(range(n_pages))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(q)[:, None, :], torch.as_tensor(keys)[None].expand(G, L, D),
        torch.as_tensor(values)[None].expand(G, L, D), scale=1 / math.sqrt(D))
    np.testing.assert_allclose(r["out"], ref[:, 0].numpy(), atol=1e-12)


def test_selected_tokens_clip_the_partial_last_page():
    L, P = 35, 16            # pages 0,1 full, page 2 holds tokens 32..34
    keys = _bf16_values((L, 8), seed=40)
    keys[33] = 50.0          # make the partial page win
    r = quest_decode_head(np.ones((1, 8)), keys, _bf16_values((L, 8), seed=41), P, 1, 0.1)
    assert r["selected"] == [2]
    np.testing.assert_array_equal(r["tokens"], [32, 33, 34])


def test_quest_decode_batched_matches_per_head():
    B, Hq, Hkv, D, P, k = 2, 8, 2, 16, 16, 3
    q = _bf16_values((B, Hq, D), seed=50)
    keys = _bf16_values((B, Hkv, 90, D), seed=51)
    values = _bf16_values((B, Hkv, 90, D), seed=52)
    lens = [90, 33]
    sel, out, lse, _ = quest_decode(q, keys, values, lens, P, k, 0.25)
    for b in range(B):
        for h in range(Hkv):
            r = quest_decode_head(q[b, 4 * h:4 * h + 4], keys[b, h, :lens[b]],
                                  values[b, h, :lens[b]], P, k, 0.25)
            n_sel = len(r["selected"])
            assert list(sel[b, h, :n_sel]) == r["selected"]
            assert all(sel[b, h, n_sel:] == -1)
            np.testing.assert_array_equal(out[b, 4 * h:4 * h + 4], r["out"])


def test_quest_decode_gqa_grouping_matches_sdpa_when_all_pages_selected():
    """With top_k >= pages, batched Quest equals dense attention in which query
    head a reads KV head a // G (torch SDPA over repeat_interleave'd heads)."""
    B, Hq, Hkv, D, P, L = 2, 8, 2, 16, 16, 70
    q = _bf16_values((B, Hq, D), seed=60)
    keys = _bf16_values((B, Hkv, L, D), seed=61)
    values = _bf16_values((B, Hkv, L, D), seed=62)
    lens = [L, 45]
    sel, out, lse, _ = quest_decode(q, keys, values, lens, P, 99, 0.25)
    ke = torch.as_tensor(keys).repeat_interleave(Hq // Hkv, dim=1)
    ve = torch.as_tensor(values).repeat_interleave(Hq // Hkv, dim=1)
    for b in range(B):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.as_tensor(q[b])[:, None, :], ke[b, :, :lens[b]], ve[b, :, :lens[b]], scale=0.25)
        np.testing.assert_allclose(out[b], ref[:, 0].numpy(), atol=1e-12)
        ref_lse = torch.logsumexp(torch.einsum("ad,atd->at", torch.as_tensor(q[b]),
                                               ke[b, :, :lens[b]]) * 0.25, dim=1)
        np.testing.assert_allclose(lse[b], ref_lse.numpy(), atol=1e-12)
