"""Pins for oracle.omnikv: token scores against a batched torch computation
(expanded GQA heads, max over heads), special cases (one head, keys on a
single axis), selection against a brute-force ranking and the pages' example
of reusing {1, 4, 8}, and the sparse layer against torch SDPA on the gathered
positions."""
import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import omnikv_select, omnikv_sparse_layer, omnikv_token_scores


@pytest.mark.parametrize("Hq,Hkv,L,D", [(8, 2, 50, 16), (4, 4, 9, 8), (32, 8, 300, 64)])
def test_token_scores_equal_batched_max_over_heads(Hq, Hkv, L, D):
    rng = np.random.default_rng(Hq + L)
    q = rng.standard_normal((Hq, D))
    k = rng.standard_normal((Hkv, L, D))
    K = torch.as_tensor(k).repeat_interleave(Hq // Hkv, dim=0)       # [Hq][L][D]
    want = torch.einsum("ald,ad->al", K, torch.as_tensor(q)).max(dim=0).values.numpy()
    np.testing.assert_allclose(omnikv_token_scores(q, k), want, rtol=1e-13, atol=1e-13)


def test_token_scores_single_head_and_axis_keys():
    q = np.array([[2.0, -1.0, 0.5]])
    k = np.array([[[1, 0, 0], [0, 1, 0], [0, 0, 1], [-1, 0, 0]]], dtype=float)
    assert omnikv_token_scores(q, k).tolist() == [2.0, -1.0, 0.5, -2.0]


@settings(max_examples=60, deadline=None)
@given(st.lists(st.integers(-3, 3), min_size=1, max_size=20), st.integers(1, 25))
def test_select_matches_brute_force(vals, b):
    got = omnikv_select(np.array(vals, dtype=float), b)
    L = len(vals)
    if L <= b:
        assert got == list(range(L))
        return
    # brute force: the set of size b with the largest score sum, lexicographically
    # smallest positions among equal sums (ties to the smaller position)
    ranked = sorted(range(L), key=lambda j: (-vals[j], j))[:b]
    assert got == sorted(ranked)
    worst_kept = min(vals[j] for j in got)
    assert all(vals[j] <= worst_kept for j in range(L) if j not in got)
    # among equal scores at the cutoff, the smaller positions are kept
    tied = [j for j in range(L) if vals[j] == worst_kept]
    kept_tied = [j for j in tied if j in got]
    assert kept_tied == tied[:len(kept_tied)]


def test_pages_example_reuse_positions_1_4_8():
    """An observation layer whose query singles out positions {1, 4, 8}
    (1-based) with budget 3 selects {0, 3, 7} (0-based); a sparse layer with
    different keys and values reads exactly those positions."""
    D, L = 8, 10
    k = np.zeros((1, L, D))
    q = np.zeros((1, D))
    q[0, 0] = 1.0
    k[0, [0, 3, 7], 0] = [3.0, 2.0, 5.0]
    sel = omnikv_select(omnikv_token_scores(q, k), 3)
    assert sel == [0, 3, 7]
    rng = np.random.default_rng(0)
    k2, v2 = rng.standard_normal((1, L, D)), rng.standard_normal((1, L, D))
    qs = rng.standard_normal((2, D))
    out, lse = omnikv_sparse_layer(qs, k2, v2, sel, 0.5)
    for a in range(2):
        z = 0.5 * k2[0][sel] @ qs[a]
        p = np.exp(z - z.max()); p /= p.sum()
        np.testing.assert_allclose(out[a], p @ v2[0][sel], rtol=1e-12)


def test_sparse_layer_equals_sdpa_on_gathered_positions():
    rng = np.random.default_rng(3)
    Hq, Hkv, L, D = 8, 2, 40, 16
    q = rng.standard_normal((Hq, D))
    k, v = rng.standard_normal((Hkv, L, D)), rng.standard_normal((Hkv, L, D))
    pos = [1, 5, 6, 20, 39]
    out, _ = omnikv_sparse_layer(q, k, v, pos, 0.25)
    K = torch.as_tensor(k[:, pos]).repeat_interleave(Hq // Hkv, 0)
    V = torch.as_tensor(v[:, pos]).repeat_interleave(Hq // Hkv, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(q)[:, None, :], K, V, scale=0.25)[:, 0]
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)
