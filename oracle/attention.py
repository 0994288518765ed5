"""Softmax attention of one query over a set of keys (fp64).

"SparseEngine: Sparse-First Inference Engine", Appendix A.1, "Attention over
Selected Positions": for a nonempty set S_i of key positions, attention
normalises over the selected positions only; dense causal attention is the
case S_i = all positions.  The display formula was lost in extraction; the
reading is standard scaled dot-product attention,
    z_j = scale * (q . k_j),  p_j = exp(z_j) / sum_{j' in S} exp(z_j'),
    o = sum_{j in S} p_j v_j,  lse = log sum_{j in S} exp(z_j),
with scale = 1/sqrt(d_k) supplied by the caller.

Appendix A.1, "MHA, MQA, and GQA": query head a reads KV head g(a); with
H_q = G * H_kv heads, g(a) = floor(a / G).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    """Exact conversion of a torch tensor / array of fp32 or bf16 values to float64."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def attend(q, keys, values, scale: float):
    """One query head over a set of tokens.

    q: [D]; keys, values: [T][D] (the tokens of S, any order).
    Returns (o [D], lse, p [T], z [T]).  T must be >= 1."""
    q = _f64(q)
    keys = _f64(keys)
    values = _f64(values)
    if keys.shape[0] == 0:
        raise ValueError("attention over an empty set is undefined")
    z = (keys @ q) * float(scale)          # logits
    m = z.max()
    w = np.exp(z - m)
    l = w.sum()
    p = w / l                               # normalised over S only
    o = p @ values
    lse = m + np.log(l)
    return o, lse, p, z


def attend_heads(qs, keys, values, scale: float):
    """The G query heads that share one KV head: qs [G][D], keys/values [T][D].
    Returns (out [G][D], lse [G], probs [G][T], logits [G][T])."""
    qs = _f64(qs)
    G = qs.shape[0]
    T = _f64(keys).shape[0]
    out = np.zeros((G, qs.shape[1]))
    lse = np.zeros(G)
    probs = np.zeros((G, T))
    logits = np.zeros((G, T))
    for a in range(G):
        out[a], lse[a], probs[a], logits[a] = attend(qs[a], keys, values, scale)
    return out, lse, probs, logits


def dense_decode(q, keys, values, lens, scale: float):
    """Dense decode attention over each sequence's first lens[b] slots.

    q [B][H_q][D]; keys, values [B][H_kv][>=max(lens)][D]; query head a of
    sequence b reads KV head a // G over slots [0, lens[b]).
    Returns (out [B][H_q][D], lse [B][H_q]); sequences with lens[b] == 0 get
    out = 0 and lse = -inf."""
    q = _f64(q)
    B, Hq, D = q.shape
    Hkv = _f64(keys[0:1]).shape[1] if hasattr(keys, "shape") else len(keys[0])
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        for h in range(Hkv):
            kb = _f64(keys[b][h][:L])
            vb = _f64(values[b][h][:L])
            for a in range(h * G, (h + 1) * G):
                out[b, a], lse[b, a], _, _ = attend(q[b, a], kb, vb, scale)
    return out, lse
