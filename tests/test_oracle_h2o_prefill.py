"""Pins for the chunk-wise H2O prefill of the oracle (oracle.h2o_prefill_chunk,
oracle.h2o_prefill): an independent masked softmax written with torch tensor
ops, closed forms under uniform attention (exact fractions), conservation of
probability mass, and the reduction of a one-token chunk to a decode step."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import H2OHeadState, h2o_prefill, h2o_prefill_chunk, h2o_retain
from oracle.h2o import h2o_append, h2o_attend_accumulate


def _state(n, D, rng):
    return H2OHeadState(np.arange(n, dtype=np.int64), rng.standard_normal((n, D)),
                        rng.standard_normal((n, D)), rng.random(n) * 3)


@pytest.mark.parametrize("n_r,n,G,D", [(0, 9, 1, 8), (5, 7, 3, 16), (40, 33, 4, 32)])
def test_chunk_scores_equal_causal_masked_softmax_in_torch(n_r, n, G, D):
    rng = np.random.default_rng(n_r + n)
    st = _state(n_r, D, rng)
    q = rng.standard_normal((n, G, D))
    kc, vc = rng.standard_normal((n, D)), rng.standard_normal((n, D))
    scale = 0.3
    got = h2o_prefill_chunk(st, q, np.arange(n_r, n_r + n), kc, vc, scale)
    # torch: logits [n*G][n_r + n], query i sees columns [0, n_r + i]
    K = torch.cat([torch.as_tensor(st.keys), torch.as_tensor(kc)])
    Q = torch.as_tensor(q).reshape(n * G, D)
    z = scale * Q @ K.T
    qi = torch.arange(n).repeat_interleave(G)[:, None]
    col = torch.arange(n_r + n)[None, :]
    z = z.masked_fill(col > n_r + qi, float("-inf"))
    add = torch.softmax(z, dim=1).sum(0).numpy()
    want = np.concatenate([st.scores, np.zeros(n)]) + add
    np.testing.assert_allclose(got.scores, want, rtol=1e-12, atol=1e-12)
    assert got.positions.tolist() == list(range(n_r + n))


def test_chunk_uniform_attention_closed_form():
    """Identical keys: chunk query i spreads 1/(n_r + i + 1) over every visible
    entry, so a retained entry gains G * sum_i 1/(n_r+i+1) and chunk entry j
    gains G * sum_{i >= j} 1/(n_r+i+1) (exact fractions)."""
    n_r, n, G, D = 6, 5, 2, 4
    rng = np.random.default_rng(1)
    st = H2OHeadState(np.arange(n_r, dtype=np.int64), np.ones((n_r, D)), rng.standard_normal((n_r, D)),
                      np.zeros(n_r))
    got = h2o_prefill_chunk(st, rng.standard_normal((n, G, D)), np.arange(n_r, n_r + n),
                            np.ones((n, D)), rng.standard_normal((n, D)), 0.7)
    for j in range(n_r + n):
        first = max(0, j - n_r)
        exact = G * sum(Fraction(1, n_r + i + 1) for i in range(first, n))
        assert abs(got.scores[j] - float(exact)) < 1e-12


def test_chunk_mass_conservation():
    rng = np.random.default_rng(2)
    st = _state(12, 8, rng)
    n, G = 9, 4
    got = h2o_prefill_chunk(st, rng.standard_normal((n, G, 8)) * 3, np.arange(12, 21),
                            rng.standard_normal((n, 8)), rng.standard_normal((n, 8)), 1.0)
    assert abs(got.scores.sum() - (st.scores.sum() + G * n)) < 1e-9


def test_one_token_chunk_is_a_decode_step():
    rng = np.random.default_rng(3)
    st = _state(10, 8, rng)
    q = rng.standard_normal((1, 3, 8))
    k, v = rng.standard_normal(8), rng.standard_normal(8)
    got = h2o_prefill_chunk(st, q, [10], k[None], v[None], 0.5)
    ref, *_ = h2o_attend_accumulate(h2o_append(st, 10, k, v), q[0], 0.5)
    np.testing.assert_allclose(got.scores, ref.scores, rtol=1e-13, atol=1e-13)


def test_prefill_without_eviction_is_full_causal_attention():
    """chunk >= n and budget >= n: the scores are the column sums of the full
    causal softmax, whatever the chunking."""
    rng = np.random.default_rng(4)
    n, G, D = 23, 2, 8
    q, k, v = rng.standard_normal((n, G, D)), rng.standard_normal((n, D)), rng.standard_normal((n, D))
    one = h2o_prefill(q, k, v, chunk=n, budget=n, window=0, scale=0.4)
    several = h2o_prefill(q, k, v, chunk=5, budget=n, window=0, scale=0.4)
    np.testing.assert_allclose(one.scores, several.scores, rtol=1e-12, atol=1e-12)
    Q = torch.as_tensor(q).reshape(n * G, D)
    z = 0.4 * Q @ torch.as_tensor(k).T
    qi = torch.arange(n).repeat_interleave(G)[:, None]
    z = z.masked_fill(torch.arange(n)[None, :] > qi, float("-inf"))
    np.testing.assert_allclose(one.scores, torch.softmax(z, 1).sum(0).numpy(), rtol=1e-12, atol=1e-12)


def test_prefill_evicts_after_every_chunk():
    """Budget 6, window 2, chunks of 4 over 12 tokens: after each chunk the
    state holds min(available, 6) entries, the window is the chunk's last two
    positions, and the kept older entries are the top scores of that moment."""
    rng = np.random.default_rng(5)
    n, G, D = 12, 2, 8
    q, k, v = rng.standard_normal((n, G, D)), rng.standard_normal((n, D)), rng.standard_normal((n, D))
    st = H2OHeadState(np.zeros(0, np.int64), np.zeros((0, D)), np.zeros((0, D)), np.zeros(0))
    for c0 in range(0, n, 4):
        acc = h2o_prefill_chunk(st, q[c0:c0 + 4], np.arange(c0, c0 + 4), k[c0:c0 + 4], v[c0:c0 + 4], 0.5)
        keep = h2o_retain(acc.positions, acc.scores, 6, 2)
        assert len(keep) == min(len(acc), 6)
        assert {c0 + 2, c0 + 3} <= set(acc.positions[keep].tolist())
        st = H2OHeadState(acc.positions[keep], acc.keys[keep], acc.values[keep], acc.scores[keep])
    final = h2o_prefill(q, k, v, chunk=4, budget=6, window=2, scale=0.5)
    assert final.positions.tolist() == st.positions.tolist()
    np.testing.assert_allclose(final.scores, st.scores)
