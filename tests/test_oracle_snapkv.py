"""Pins for oracle.snapkv: an independent masked-softmax computation in torch
float64, a closed form for uniform attention, pooling against torch's
max_pool1d and a hand-worked example, the pages' eight-token example, and
brute force over retained sets."""
import itertools

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import snapkv_window_scores, snapkv_pool, snapkv_retain


def _vals(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("n,w,G,D", [(40, 4, 2, 16), (100, 32, 4, 32), (33, 32, 1, 8), (9, 1, 3, 4)])
def test_window_scores_equal_masked_softmax_in_torch(n, w, G, D):
    keys = _vals((n, D), seed=n + w)
    q = _vals((w, G, D), seed=n * 3 + G)
    scale = 1.0 / np.sqrt(D)
    u = snapkv_window_scores(q, keys, scale)
    # one logits matrix for all (query, head) rows, causal mask, torch softmax
    Q = torch.tensor(q).reshape(w * G, D)                # row i*G + a
    K = torch.tensor(keys)
    z = scale * (Q @ K.T)
    pos = torch.arange(w).repeat_interleave(G) + (n - w)
    z = z.masked_fill(torch.arange(n)[None, :] > pos[:, None], float("-inf"))
    p = torch.softmax(z, dim=1)
    expect = p[:, :n - w].sum(0).numpy()
    np.testing.assert_allclose(u, expect, rtol=0, atol=1e-12)


def test_window_scores_uniform_attention_closed_form():
    n, w, G = 50, 6, 3
    keys = np.zeros((n, 8))
    q = _vals((w, G, 8), seed=1)
    u = snapkv_window_scores(q, keys, 0.3)
    # every logit is 0: query i spreads 1 / (n - w + i + 1) on each visible position
    expect = sum(G / (n - w + i + 1) for i in range(w))
    np.testing.assert_allclose(u, np.full(n - w, expect), rtol=1e-14)


def test_window_scores_single_query_loop_form():
    n, D = 20, 6
    keys = _vals((n, D), seed=7)
    q = _vals((1, 1, D), seed=8)
    u = snapkv_window_scores(q, keys, 0.5)
    z = [0.5 * sum(float(keys[j, c]) * float(q[0, 0, c]) for c in range(D)) for j in range(n)]
    den = sum(np.exp(v) for v in z)
    for j in range(n - 1):
        assert abs(u[j] - np.exp(z[j]) / den) < 1e-14


@pytest.mark.parametrize("kernel", [1, 3, 5, 7, 9, 15])
@pytest.mark.parametrize("n", [1, 4, 37, 200])
def test_pool_matches_torch_max_pool1d(kernel, n):
    """An odd kernel centred at j with the edges clipped is torch's max_pool1d
    with stride 1 and kernel // 2 of (implicit -inf) padding on both sides."""
    u = _vals((n,), seed=kernel * 1000 + n)
    s = snapkv_pool(u, kernel)
    t = torch.nn.functional.max_pool1d(torch.tensor(u)[None, None], kernel_size=kernel, stride=1,
                                       padding=kernel // 2)[0, 0].numpy()
    np.testing.assert_array_equal(s, t)
    if kernel == 1:
        np.testing.assert_array_equal(s, u)


@pytest.mark.parametrize("kernel", [2, 4])
def test_pool_even_kernel_is_the_next_odd_window(kernel):
    """Reading for an even width: the neighbourhood [j - kernel/2, j + kernel/2]
    (kernel + 1 positions) centred at j, i.e. torch's odd window kernel + 1."""
    u = _vals((41,), seed=kernel)
    t = torch.nn.functional.max_pool1d(torch.tensor(u)[None, None], kernel_size=kernel + 1, stride=1,
                                       padding=kernel // 2)[0, 0].numpy()
    np.testing.assert_array_equal(snapkv_pool(u, kernel), t)


def test_pool_hand_worked_clipped_edges():
    """Worked by hand: u = 5 1 0 2 9 3 4 0.  Width 3 takes each position with
    its two neighbours (one at the ends); width 7 takes three on each side, so
    position 1 already sees the 9 at position 4, and position 0 sees 0..3."""
    u = [5.0, 1.0, 0.0, 2.0, 9.0, 3.0, 4.0, 0.0]
    assert snapkv_pool(u, 3).tolist() == [5.0, 5.0, 2.0, 9.0, 9.0, 9.0, 4.0, 4.0]
    assert snapkv_pool(u, 7).tolist() == [5.0, 9.0, 9.0, 9.0, 9.0, 9.0, 9.0, 9.0]
    assert snapkv_pool(u, 1).tolist() == u
    # a single earlier position: every width returns it
    assert snapkv_pool([-2.5], 7).tolist() == [-2.5]


def test_retain_eight_token_example():
    """Eight-token prompt, w = 2, B = 4: positions 7 and 8 (1-based) plus the
    two earlier positions with the largest pooled scores."""
    pooled = np.array([0.1, 0.9, 0.3, 0.8, 0.2, 0.05])
    assert snapkv_retain(8, pooled, budget=4, window=2) == [1, 3, 6, 7]


def _brute_force_retain(n, pooled, budget, window, n_sink):
    earlier = range(n - window)
    fixed = set(range(n - window, n)) | set(range(min(n_sink, n - window)))
    best = None
    for sub in itertools.combinations([j for j in earlier if j not in fixed], budget - len(fixed)):
        key = sorted(((pooled[j], -j) for j in sub), reverse=True)
        if best is None or key > best[0]:
            best = (key, sub)
    return sorted(fixed | set(best[1]))


@settings(max_examples=150, deadline=None)
@given(st.integers(4, 9), st.integers(0, 3), st.integers(0, 2), st.data())
def test_retain_brute_force(n, window, n_sink, data):
    if window + n_sink > n:
        return                            # the budget must hold the window and the sinks
    budget = data.draw(st.integers(window + n_sink, n))
    pooled = [float(v) for v in data.draw(st.lists(st.integers(-2, 2), min_size=n - window,
                                                     max_size=n - window))]
    got = snapkv_retain(n, pooled, budget, window, n_sink)
    if n <= budget:
        assert got == list(range(n))
    else:
        assert got == _brute_force_retain(n, pooled, budget, window, n_sink)


def test_retain_keeps_everything_within_budget_and_sinks_always():
    assert snapkv_retain(5, [0.0] * 3, budget=5, window=2) == [0, 1, 2, 3, 4]
    pooled = np.arange(20.0)              # later positions score higher
    kept = snapkv_retain(24, pooled, budget=10, window=4, n_sink=2)
    assert kept[:2] == [0, 1] and kept[-4:] == [20, 21, 22, 23] and len(kept) == 10
    assert kept[2:6] == [16, 17, 18, 19]
