"""Pins for oracle.h2o: closed forms under uniform attention (exact rational
arithmetic), conservation of probability mass, property checks that fix the
retained set uniquely, and the pages' budget-4 / two-recent example."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import H2OHeadState, h2o_retain, h2o_step_head
from oracle.h2o import h2o_attend_accumulate, h2o_append

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _empty(D):
    return H2OHeadState(np.zeros(0, dtype=np.int64), np.zeros((0, D)), np.zeros((0, D)),
                        np.zeros(0))


def test_budget4_two_recent_example_uniform_attention():
    """With q = 0 every query spreads weight 1/n over the n available tokens,
    so each step adds exactly G/n to every resident score (exact fractions
    below, independent of the oracle's softmax).  Budget 4, window 2, G = 2:
      step 0..3: no eviction (n <= 4)
      step 4: n = 5, window = positions {3, 4}; the older three compete and the
              lowest-scoring one (position 2) is evicted
      step 5: position 3 leaves the window and now competes on its score; it
              is the lowest of {0, 1, 3} and is evicted."""
    with open(os.path.join(GOLDEN, "h2o_budget4_two_recent.json")) as f:
        ex = json.load(f)
    B, W, G, D = ex["budget"], ex["recent_window"], 2, 4
    state = _empty(D)
    exact = {}                     # position -> Fraction score
    kept_expected = []
    for i in range(7):
        exact[i] = Fraction(0)
        n = len(exact)
        for pos in exact:
            exact[pos] += Fraction(G, n)
        if n > B:
            by_pos = sorted(exact)
            win = by_pos[-W:]
            rest = sorted(by_pos[:-W], key=lambda p: (-exact[p], p))[:B - W]
            exact = {p: exact[p] for p in sorted(win + rest)}
        kept_expected.append(sorted(exact))
        state, _, _, _, _ = h2o_step_head(state, np.zeros((G, D)), i, np.ones(D) * i,
                                          np.arange(D) + i, B, W, 1.0)
        assert list(state.positions) == kept_expected[-1]
        np.testing.assert_allclose(state.scores, [float(exact[p]) for p in state.positions],
                                   rtol=0, atol=1e-14)
    assert kept_expected[4] == [0, 1, 3, 4]        # position 2 evicted at step 4
    assert kept_expected[5] == [0, 1, 4, 5]        # position 3 left the window, evicted
    # payload rows follow their positions
    for j, p in enumerate(state.positions):
        np.testing.assert_array_equal(state.keys[j], np.ones(D) * p)
        np.testing.assert_array_equal(state.values[j], np.arange(D) + p)


def test_new_token_enters_with_score_zero_then_gets_its_mass():
    g = torch.Generator().manual_seed(3)
    D, G = 16, 4
    st0 = H2OHeadState.from_arrays(np.arange(5), torch.randn(5, D, generator=g),
                                   torch.randn(5, D, generator=g), np.arange(5) * 0.1)
    app = h2o_append(st0, 9, torch.randn(D, generator=g), torch.randn(D, generator=g))
    assert app.scores[-1] == 0.0
    qs = torch.randn(G, D, generator=g, dtype=torch.float64)
    acc, _, _, _, probs = h2o_attend_accumulate(app, qs, 0.25)
    assert acc.scores[-1] == pytest.approx(probs[:, -1].sum(), abs=0)
    # the new token's mass equals SDPA-style softmax weight from torch.softmax
    keys = torch.as_tensor(app.keys)
    w = torch.softmax((qs @ keys.T) * 0.25, dim=1)
    assert acc.scores[-1] == pytest.approx(float(w[:, -1].sum()), abs=1e-14)
    np.testing.assert_allclose(acc.scores, app.scores + w.sum(0).numpy(), atol=1e-14)


@pytest.mark.parametrize("G", [1, 4, 8])
def test_accumulate_conserves_mass(G):
    g = torch.Generator().manual_seed(G)
    D, n = 32, 77
    st0 = H2OHeadState.from_arrays(np.arange(n), torch.randn(n, D, generator=g),
                                   torch.randn(n, D, generator=g),
                                   torch.rand(n, generator=g, dtype=torch.float64))
    acc, _, _, _, probs = h2o_attend_accumulate(st0, torch.randn(G, D, generator=g), 0.2)
    assert acc.scores.sum() == pytest.approx(st0.scores.sum() + G, abs=1e-12)
    np.testing.assert_allclose(probs.sum(axis=1), np.ones(G), atol=1e-14)


def _check_retained(positions, scores, budget, window, keep):
    n = len(positions)
    assert len(keep) == min(n, budget)
    assert [positions[j] for j in keep] == sorted(positions[j] for j in keep)
    if n <= budget:
        assert keep == list(range(n))
        return
    order = sorted(range(n), key=lambda j: positions[j])
    win = set(order[n - window:]) if window > 0 else set()
    assert win <= set(keep)
    kept_rest = [j for j in keep if j not in win]
    dropped = [j for j in range(n) if j not in set(keep)]
    for a in kept_rest:
        for d in dropped:
            assert scores[a] > scores[d] or (scores[a] == scores[d] and positions[a] < positions[d])


@settings(max_examples=300, deadline=None)
@given(st.lists(st.integers(0, 4), min_size=1, max_size=12), st.integers(1, 8), st.data())
def test_retain_properties_with_ties(score_ints, budget, data):
    n = len(score_ints)
    window = data.draw(st.integers(0, budget))
    positions = sorted(data.draw(st.lists(st.integers(0, 100), min_size=n, max_size=n,
                                          unique=True)))
    scores = [float(s) for s in score_ints]
    keep = h2o_retain(positions, scores, budget, window)
    _check_retained(positions, scores, budget, window, keep)


def test_retain_brute_force_small():
    """Every subset of size budget that contains the window; the retained one
    maximises the descending list of (score, -position) of its non-window part."""
    import itertools
    rng = np.random.default_rng(7)
    for trial in range(200):
        n = int(rng.integers(2, 9))
        budget = int(rng.integers(1, n))
        window = int(rng.integers(0, budget + 1))
        positions = sorted(rng.choice(50, n, replace=False).tolist())
        scores = rng.integers(0, 3, n).astype(float).tolist()
        win = set(range(n - window, n))
        best = None
        for sub in itertools.combinations(range(n), budget):
            if not win <= set(sub):
                continue
            key = sorted(((scores[j], -positions[j]) for j in sub if j not in win), reverse=True)
            if best is None or key > best[0]:
                best = (key, list(sub))
        assert h2o_retain(positions, scores, budget, window) == best[1]


def test_retain_window_equal_budget_keeps_only_recent():
    keep = h2o_retain([0, 2, 5, 9, 11], [9.0, 8.0, 7.0, 0.0, 0.0], 2, 2)
    assert keep == [3, 4]


def test_retain_rejects_window_above_budget():
    with pytest.raises(ValueError):
        h2o_retain([0, 1, 2], [0.0, 0.0, 0.0], 1, 2)


def test_free_running_invariants():
    g = torch.Generator().manual_seed(11)
    D, G, budget, W = 16, 4, 12, 3
    state = H2OHeadState.from_arrays(np.arange(20), torch.randn(20, D, generator=g),
                                     torch.randn(20, D, generator=g), np.zeros(20))
    orig_k = {int(p): state.keys[j].copy() for j, p in enumerate(state.positions)}
    for i in range(20, 40):
        kn, vn = torch.randn(D, generator=g), torch.randn(D, generator=g)
        orig_k[i] = kn.double().numpy()
        before = state.scores.sum()
        state, _, _, acc_scores, _ = h2o_step_head(state, torch.randn(G, D, generator=g), i,
                                                   kn, vn, budget, W, 0.25)
        assert acc_scores.sum() == pytest.approx(before + G, abs=1e-11)
        assert len(state) == budget
        assert np.all(np.diff(state.positions) > 0)
        assert list(state.positions[-W:]) == list(range(i - W + 1, i + 1))
        for j, p in enumerate(state.positions):
            np.testing.assert_array_equal(state.keys[j], orig_k[int(p)])
