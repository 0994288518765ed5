"""OmniKV cross-layer token-index reuse for one sequence (fp64).

"SparseEngine: Sparse-First Inference Engine", Appendix A.3, "OmniKV":
designated observation (filter) layers inspect the context during decoding
and produce token indices that the sparse layers assigned to them reuse; a
current-query selector ranks every position by its largest query-key logit
across heads and keeps the selected-token budget b (formula lost; read as
r(j) = max over query heads a of q_a . k_{g(a), j} and the b positions with
the largest r).  A sparse layer reads those positions from its own cache and
computes its own attention over them (Appendix A.1, attention over a set).

Readings where the pages are silent:
  * the maximum runs over every query head of the layer, each head reading
    its own KV head (GQA, Appendix A.1), so one index set serves the whole
    sequence and every KV head of the sparse layers;
  * logits are ranked unscaled (a positive temperature does not change the
    order); ties keep the smaller position; the kept positions are listed
    in ascending order; when L <= b every position is kept.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, attend


def omnikv_token_scores(q, keys):
    """r(j) for one sequence: q [H_q][D], keys [H_kv][L][D]; query head a
    reads KV head a // (H_q / H_kv).  Returns r [L]."""
    q = _f64(q)
    keys = _f64(keys)
    Hq = q.shape[0]
    Hkv, L, _ = keys.shape
    G = Hq // Hkv
    r = np.full(L, -np.inf)
    for a in range(Hq):
        r = np.maximum(r, keys[a // G] @ q[a])
    return r


def omnikv_select(scores, budget: int):
    """Positions (ascending) of the `budget` largest scores, ties to the
    smaller position; every position when there are at most `budget`."""
    scores = np.asarray(scores, dtype=np.float64)
    L = len(scores)
    if L <= budget:
        return list(range(L))
    order = sorted(range(L), key=lambda j: (-scores[j], j))
    return sorted(order[:budget])


def omnikv_sparse_layer(q, keys, values, positions, scale: float):
    """A sparse layer's attention over the reused positions of its own cache:
    q [H_q][D], keys/values [H_kv][L][D].  Returns (out [H_q][D], lse [H_q])."""
    q = _f64(q)
    keys, values = _f64(keys), _f64(values)
    Hq, D = q.shape
    G = Hq // keys.shape[0]
    pos = np.asarray(positions, dtype=np.int64)
    out = np.zeros((Hq, D))
    lse = np.zeros(Hq)
    for a in range(Hq):
        out[a], lse[a], _, _ = attend(q[a], keys[a // G][pos], values[a // G][pos], scale)
    return out, lse
