"""H2O accumulated-score eviction for one (sequence, KV head) (fp64).

"SparseEngine: Sparse-First Inference Engine", Appendix A.3, "H2O: Accumulated
Scores and Online Eviction":
  * before processing position i the available set is A_i = R_{i-1} + {i};
  * attention reads A_i and its weights are added to persistent per-token
    scores, the new token starting from zero before this update (update
    formula lost in extraction; read as s_j <- s_j + p_j for j in A_i);
  * with cache budget B and a protected recent window W_i of at most B
    positions, the retained set R_i is the window plus the highest-scoring
    other positions (formula lost; read as the W largest positions of A_i plus
    the top B - W of the rest by score), evicting everything else while the
    retained entries keep their scores.
Section 3.1, "Architectural Foundations": physical eviction rewrites the
retained-slot mapping and the context length.

Readings where the pages are silent:
  * GQA: one retained set per KV head, scored by the sum over the group's
    query heads of their attention probabilities;
  * eviction runs after attention in the same step, only when |A_i| > B;
  * ties among equal scores keep the smaller position;
  * retained entries stay in ascending position order (order-preserving
    compaction), so the window is the last W entries.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .attention import _f64, attend


@dataclasses.dataclass
class H2OHeadState:
    """Retained entries of one (sequence, KV head), in ascending position."""
    positions: np.ndarray      # [n] int64
    keys: np.ndarray           # [n][D] float64
    values: np.ndarray         # [n][D] float64
    scores: np.ndarray         # [n] float64

    @classmethod
    def from_arrays(cls, positions, keys, values, scores):
        return cls(np.asarray(positions, dtype=np.int64).copy(), _f64(keys).copy(),
                   _f64(values).copy(), np.asarray(_f64(scores), dtype=np.float64).copy())

    def copy(self):
        return H2OHeadState(self.positions.copy(), self.keys.copy(), self.values.copy(),
                            self.scores.copy())

    def __len__(self):
        return len(self.positions)


def h2o_retain(positions, scores, budget: int, window: int):
    """Indices (into the given arrays, ascending position) of the entries kept
    when shrinking to ``budget``: the ``window`` entries with the largest
    positions, plus the top ``budget - window`` of the others by
    (score descending, position ascending).  Requires 0 <= window <= budget."""
    positions = np.asarray(positions)
    scores = np.asarray(scores, dtype=np.float64)
    n = len(positions)
    if not (0 <= window <= budget):
        raise ValueError("need 0 <= window <= budget")
    if n <= budget:
        return list(range(n))
    by_pos_desc = sorted(range(n), key=lambda j: -int(positions[j]))
    win = set(by_pos_desc[:window])
    rest = [j for j in range(n) if j not in win]
    ranked = sorted(rest, key=lambda j: (-scores[j], int(positions[j])))
    keep = win | set(ranked[:budget - window])
    return sorted(keep, key=lambda j: int(positions[j]))


def h2o_append(state: H2OHeadState, position: int, k_new, v_new) -> H2OHeadState:
    """A_i = R_{i-1} + {i}: the new token enters with score zero."""
    return H2OHeadState(
        np.append(state.positions, np.int64(position)),
        np.vstack([state.keys, _f64(k_new)[None, :]]),
        np.vstack([state.values, _f64(v_new)[None, :]]),
        np.append(state.scores, 0.0))


def h2o_attend_accumulate(state: H2OHeadState, qs, scale: float):
    """Attention of the group's query heads over every entry, then
    s_j += sum_a p_{a,j}.  Returns (new state, out [G][D], lse [G],
    logits [G][n], probs [G][n])."""
    qs = _f64(qs)
    G, D = qs.shape
    n = len(state)
    out = np.zeros((G, D))
    lse = np.zeros(G)
    logits = np.zeros((G, n))
    probs = np.zeros((G, n))
    scores = state.scores.copy()
    for a in range(G):
        out[a], lse[a], probs[a], logits[a] = attend(qs[a], state.keys, state.values, scale)
        scores = scores + probs[a]
    new = H2OHeadState(state.positions.copy(), state.keys.copy(), state.values.copy(), scores)
    return new, out, lse, logits, probs


def h2o_evict(state: H2OHeadState, budget: int, window: int) -> H2OHeadState:
    """Keep R_i (see h2o_retain); everything else is dropped."""
    keep = h2o_retain(state.positions, state.scores, budget, window)
    return H2OHeadState(state.positions[keep], state.keys[keep], state.values[keep],
                        state.scores[keep])


def h2o_step_head(state: H2OHeadState, qs, position: int, k_new, v_new, budget: int,
                  window: int, scale: float):
    """One decode step: append, attend + accumulate, evict.
    Returns (new state, out [G][D], lse [G], scores after accumulation
    (before eviction, aligned with the appended state), appended state)."""
    appended = h2o_append(state, position, k_new, v_new)
    acc, out, lse, _, _ = h2o_attend_accumulate(appended, qs, scale)
    new = h2o_evict(acc, budget, window)
    return new, out, lse, acc.scores, appended


def h2o_prefill_chunk(state: H2OHeadState, q_chunk, positions, k_chunk, v_chunk, scale: float):
    """One prefill chunk for one (sequence, KV head).

    SE Appendix A.3 "H2O" with the chunk-wise prefill of SE Section 3.1
    ("Fine-Grained Lifecycle Hooks"): the chunk's n tokens join the available
    set with score zero; every chunk query attends over the retained entries
    and the chunk's entries up to its own position (causal), and its
    probabilities are added to the scores.  q_chunk [n][G][D] (the group's
    query heads), positions [n] above every retained position.  Returns the
    state after accumulation, before any eviction."""
    q_chunk = _f64(q_chunk)
    n, G, _ = q_chunk.shape
    positions = np.asarray(positions, dtype=np.int64)
    keys = np.vstack([state.keys, _f64(k_chunk)])
    values = np.vstack([state.values, _f64(v_chunk)])
    pos = np.concatenate([state.positions, positions])
    scores = np.concatenate([state.scores, np.zeros(n)])
    n_r = len(state)
    for i in range(n):
        vis = n_r + i + 1                       # retained entries, then the chunk up to query i
        for a in range(G):
            z = scale * (keys[:vis] @ q_chunk[i, a])
            p = np.exp(z - z.max())
            scores[:vis] += p / p.sum()
    return H2OHeadState(pos, keys, values, scores)


def h2o_prefill(q, keys, values, chunk: int, budget: int, window: int, scale: float):
    """Chunked prefill of one (sequence, KV head) prompt: q [n][G][D],
    keys/values [n][D] in position order.  After every chunk the scores are
    accumulated (h2o_prefill_chunk) and the cache is evicted down to the
    budget (h2o_evict).  Returns the final state."""
    q = _f64(q)
    keys, values = _f64(keys), _f64(values)
    n, _, D = q.shape
    state = H2OHeadState(np.zeros(0, np.int64), np.zeros((0, D)), np.zeros((0, D)), np.zeros(0))
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        state = h2o_prefill_chunk(state, q[c0:c1], np.arange(c0, c1), keys[c0:c1], values[c0:c1], scale)
        state = h2o_evict(state, budget, window)
    return state
