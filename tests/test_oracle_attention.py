"""Pins for oracle.attention: independent library routine (torch SDPA in
float64), closed forms, and the pages' subset example."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attend, attend_heads, dense_decode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sdpa(q, k, v, scale):
    # q [D], k/v [T][D] -> output via torch's own SDPA in float64
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(q, dtype=torch.float64)[None, None, None, :],
        torch.as_tensor(k, dtype=torch.float64)[None, None],
        torch.as_tensor(v, dtype=torch.float64)[None, None], scale=scale)
    return o[0, 0, 0].numpy()


@pytest.mark.parametrize("T,D", [(1, 8), (7, 16), (64, 64), (300, 128)])
def test_attend_matches_torch_sdpa(T, D):
    g = torch.Generator().manual_seed(T * 31 + D)
    q = torch.randn(D, generator=g, dtype=torch.float64)
    k = torch.randn(T, D, generator=g, dtype=torch.float64)
    v = torch.randn(T, D, generator=g, dtype=torch.float64)
    scale = 1.0 / math.sqrt(D)
    o, lse, p, z = attend(q, k, v, scale)
    np.testing.assert_allclose(o, _sdpa(q, k, v, scale), rtol=0, atol=1e-12)
    # lse against torch.logsumexp of the scaled logits
    ref_lse = torch.logsumexp((k @ q) * scale, 0).item()
    assert abs(lse - ref_lse) < 1e-12
    assert abs(p.sum() - 1.0) < 1e-12


def test_attend_zero_query_is_mean_of_values():
    g = torch.Generator().manual_seed(5)
    k = torch.randn(11, 32, generator=g, dtype=torch.float64)
    v = torch.randn(11, 32, generator=g, dtype=torch.float64)
    o, lse, p, _ = attend(torch.zeros(32, dtype=torch.float64), k, v, 0.3)
    np.testing.assert_allclose(o, v.numpy().mean(axis=0), atol=1e-14)
    assert abs(lse - math.log(11)) < 1e-14
    np.testing.assert_allclose(p, np.full(11, 1 / 11), atol=1e-15)


def test_attend_identical_keys_is_mean_of_values():
    g = torch.Generator().manual_seed(6)
    row = torch.randn(16, generator=g, dtype=torch.float64)
    k = row[None, :].repeat(9, 1)
    v = torch.randn(9, 16, generator=g, dtype=torch.float64)
    q = torch.randn(16, generator=g, dtype=torch.float64)
    o, lse, _, _ = attend(q, k, v, 0.25)
    np.testing.assert_allclose(o, v.numpy().mean(axis=0), atol=1e-13)
    assert abs(lse - (0.25 * float(row @ q) + math.log(9))) < 1e-12


def test_attend_dominant_token_returns_its_value():
    # one logit 200 above the rest: softmax is one-hot to double precision
    k = np.zeros((5, 4)); k[3, 0] = 1.0
    v = np.arange(20, dtype=np.float64).reshape(5, 4)
    q = np.array([200.0, 0, 0, 0])
    o, lse, _, _ = attend(q, k, v, 1.0)
    np.testing.assert_allclose(o, v[3], atol=1e-12)
    assert abs(lse - 200.0) < 1e-12


def test_subset_renormalisation_example():
    """Reading {1,4,8} of an eight-token cache: the result is the dense softmax
    restricted to those positions and renormalised (computed here from
    torch.softmax over all eight, not from the oracle)."""
    with open(os.path.join(GOLDEN, "subset_of_eight.json")) as f:
        ex = json.load(f)
    n = ex["cache_tokens"]
    sel = [j - 1 for j in ex["selected_positions_1based"]]
    g = torch.Generator().manual_seed(8)
    q = torch.randn(16, generator=g, dtype=torch.float64)
    k = torch.randn(n, 16, generator=g, dtype=torch.float64)
    v = torch.randn(n, 16, generator=g, dtype=torch.float64)
    full = torch.softmax((k @ q) * 0.25, 0)
    w = full[sel] / full[sel].sum()
    expect = (w[:, None] * v[sel]).sum(0).numpy()
    o, _, p, _ = attend(q, k[sel], v[sel], 0.25)
    np.testing.assert_allclose(o, expect, atol=1e-13)
    np.testing.assert_allclose(p, w.numpy(), atol=1e-14)


def test_dense_decode_gqa_grouping_matches_sdpa_with_expanded_heads():
    """Query head a reads KV head a // G: checked against torch SDPA over KV
    heads expanded with repeat_interleave."""
    B, Hq, Hkv, D, L = 2, 8, 2, 32, 40
    g = torch.Generator().manual_seed(9)
    q = torch.randn(B, Hq, D, generator=g, dtype=torch.float64)
    k = torch.randn(B, Hkv, L, D, generator=g, dtype=torch.float64)
    v = torch.randn(B, Hkv, L, D, generator=g, dtype=torch.float64)
    lens = [L, 17]
    out, lse = dense_decode(q, k, v, lens, 1 / math.sqrt(D))
    ke = k.repeat_interleave(Hq // Hkv, dim=1)
    ve = v.repeat_interleave(Hq // Hkv, dim=1)
    for b in range(B):
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[b][:, None, :], ke[b, :, :lens[b]], ve[b, :, :lens[b]], scale=1 / math.sqrt(D))
        np.testing.assert_allclose(out[b], ref[:, 0].numpy(), atol=1e-12)


def test_dense_decode_empty_sequence():
    q = np.ones((1, 2, 4)); k = np.zeros((1, 1, 3, 4)); v = np.zeros((1, 1, 3, 4))
    out, lse = dense_decode(q, k, v, [0], 1.0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_attend_heads_stacks_single_heads():
    g = torch.Generator().manual_seed(10)
    qs = torch.randn(4, 8, generator=g, dtype=torch.float64)
    k = torch.randn(6, 8, generator=g, dtype=torch.float64)
    v = torch.randn(6, 8, generator=g, dtype=torch.float64)
    out, lse, probs, logits = attend_heads(qs, k, v, 0.5)
    for a in range(4):
        np.testing.assert_allclose(out[a], _sdpa(qs[a], k, v, 0.5), atol=1e-13)
        np.testing.assert_allclose(logits[a], (k @ qs[a]).numpy() * 0.5, atol=1e-14)
