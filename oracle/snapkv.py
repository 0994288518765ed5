"""SnapKV prompt selection from an observation window (fp64).

"SparseEngine: Sparse-First Inference Engine", Appendix A.3, "SnapKV: Prompt
Selection from an Observation Window":
  * the observation window is the prompt's final w positions; every earlier
    prompt position accumulates the attention it receives from these
    observation queries (formula lost in extraction; read as
    u(j) = sum_{i in window} softmax_i(j), each observation query's softmax
    taken over its causal prefix, i.e. the positions up to its own);
  * neighbouring scores are pooled with a one-dimensional operator of width
    kappa, for example max pooling s(j) = max_{r in N(j)} u(r) over the
    prefix neighbourhood centred at j (read as r in [j - kappa//2,
    j + kappa//2] clipped to the earlier positions);
  * for a prompt-cache budget B >= w the retained prompt is the window plus
    the B - w earlier positions with the largest pooled scores (formula lost;
    the eight-token example with w = 2 and B = 4 keeps positions 7 and 8 plus
    two earlier ones); selection is per attention head.
Appendix C.1 (settings): probability-based prefill scoring with FP32 scores.
Section 5: the baseline configuration uses a scoring window of 32 and a
pooling kernel of 7 (and, for Tangram, 64 sink tokens).

Readings where the pages are silent:
  * GQA: one retained set per KV head, scored by the sum over the group's
    query heads (as for H2O);
  * softmax temperature 1/sqrt(d_k), as for decode attention;
  * optional sink tokens: the first n_sink earlier positions are always kept,
    inside the budget B;
  * ties among equal pooled scores keep the smaller position; retained
    entries stay in ascending position order.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).
"""
from __future__ import annotations

import numpy as np

from .attention import _f64


def snapkv_window_scores(q_obs, keys, scale: float):
    """u(j) for the earlier positions j < n - w of one (sequence, KV head).

    q_obs [w][G][D]: the observation queries of the group's query heads, for
    positions n - w .. n - 1 (0-based); keys [n][D] in position order.
    Returns u [n - w]."""
    q_obs = _f64(q_obs)
    keys = _f64(keys)
    w, G, _ = q_obs.shape
    n = keys.shape[0]
    u = np.zeros(n - w)
    for i in range(w):
        pos = n - w + i                      # this query sees positions 0 .. pos
        for a in range(G):
            z = scale * (keys[:pos + 1] @ q_obs[i, a])
            m = z.max()
            p = np.exp(z - m)
            p = p / p.sum()
            u += p[:n - w]
    return u


def snapkv_pool(u, kernel: int):
    """Max pooling: s(j) = max of u over [j - kernel//2, j + kernel//2]
    clipped to [0, len(u))."""
    u = np.asarray(u, dtype=np.float64)
    r = kernel // 2
    return np.array([u[max(0, j - r): j + r + 1].max() for j in range(len(u))])


def snapkv_retain(n: int, pooled, budget: int, window: int, n_sink: int = 0):
    """Positions kept of a prompt of n positions (ascending): the last
    `window`, the first n_sink earlier ones, and the best of the other earlier
    positions by pooled score (ties: smaller position) up to `budget` in all.
    Everything is kept when n <= budget.  Requires window + n_sink <= budget."""
    if not (0 <= window and window + n_sink <= budget):
        raise ValueError("need window + n_sink <= budget")
    if n <= budget:
        return list(range(n))
    w = min(window, n)
    earlier = list(range(n - w))
    pooled = np.asarray(pooled, dtype=np.float64)
    sinks = earlier[:n_sink]
    rest = sorted(earlier[n_sink:], key=lambda j: (-pooled[j], j))
    keep = set(range(n - w, n)) | set(sinks) | set(rest[:budget - w - len(sinks)])
    return sorted(keep)
