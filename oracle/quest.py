"""Quest query-dependent page selection and attention over the selected pages (fp64).

"SparseEngine: Sparse-First Inference Engine", Appendix A.3, "Quest:
Query-Dependent Page Selection":
  * token positions are grouped into pages; each page stores, per channel c,
    the minimum and the maximum key value over its tokens (formula lost in
    extraction; read as the elementwise min and max over the page's valid
    tokens);
  * a page's importance for query q upper-bounds q . k for every token k in
    the page, and need not equal any token's logit because channels can reach
    their extrema at different tokens (formula lost; read as
    U(p) = sum_c max(q_c * m_{p,c}, q_c * M_{p,c}), which has exactly those two
    properties, unscaled since a positive scale does not change the ranking);
  * pages are ranked by the estimate and attention uses the real KV of the
    selected pages; unselected pages stay stored.
Appendix A.2, "Logical Positions and Physical Blocks": with blocks of p
tokens, position j (1-based) lies in block floor((j-1)/p); 0-based here,
token t lies in page t // P.

Readings where the pages are silent:
  * GQA: selection is per KV head, with the group's per-query-head bounds
    summed, S_h(p) = sum_{a: g(a)=h} U_a(p) (reduce="sum"); the variant
    reduce="max" ranks by the largest head bound, max_{a: g(a)=h} U_a(p);
  * candidates are all ceil(L/P) pages, including the partial last page that
    holds the newest token;
  * top-k ranks by (score descending, page index ascending) and returns the
    chosen pages in ascending order; if k >= N_p every page is chosen.

Section 5 of the same page lists a Quest baseline with 16-token pages, 4 sink
pages, 32 recent pages and 92 selected pages (selected budgets exclude the
sink and recent ones).  Read as: the first n_sink pages and the last n_recent
pages (the partial last page counts) are always chosen, and the remaining
top_k - (number of forced pages) are the best of the other pages; top_k is
the total, so 4 + 32 + 92 = 128.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, attend


def page_extrema(keys, page_size: int):
    """keys [L][D] of one KV head in position order.
    Returns (mins [N_p][D], maxs [N_p][D]) with N_p = ceil(L / page_size);
    page p covers tokens [p*P, min(L, (p+1)*P))."""
    keys = _f64(keys)
    L, D = keys.shape
    n_pages = -(-L // page_size)
    mins = np.empty((n_pages, D))
    maxs = np.empty((n_pages, D))
    for p in range(n_pages):
        tok = keys[p * page_size: min(L, (p + 1) * page_size)]
        mins[p] = tok.min(axis=0)
        maxs[p] = tok.max(axis=0)
    return mins, maxs


def page_bound(q, mins, maxs):
    """U(p) = sum_c max(q_c * m_{p,c}, q_c * M_{p,c}) for every page.  q [D]."""
    q = _f64(q)
    return np.maximum(q[None, :] * mins, q[None, :] * maxs).sum(axis=1)


def group_bound(qs, mins, maxs, reduce: str = "sum"):
    """S_h(p) over the group's query heads a: the sum of U_a(p) ("sum") or
    its largest term ("max").  qs [G][D]."""
    qs = _f64(qs)
    per_head = [page_bound(qs[a], mins, maxs) for a in range(qs.shape[0])]
    if reduce == "sum":
        total = np.zeros(mins.shape[0])
        for u in per_head:
            total = total + u
        return total
    if reduce == "max":
        best = per_head[0].copy()
        for u in per_head[1:]:
            best = np.maximum(best, u)
        return best
    raise ValueError("reduce must be 'sum' or 'max'")


def forced_pages(n_pages: int, n_sink: int = 0, n_recent: int = 0):
    """Pages always chosen: the first n_sink and the last n_recent of n_pages."""
    sink = range(min(n_sink, n_pages))
    recent = range(max(0, n_pages - n_recent), n_pages)
    return sorted(set(sink) | set(recent))


def select_top_pages(scores, top_k: int, forced=()):
    """The forced pages plus the best of the others, min(top_k, N) pages in
    all: ranked by (score descending, page index ascending), returned in
    ascending page order.  Requires len(forced) <= top_k."""
    scores = np.asarray(scores, dtype=np.float64)
    forced = sorted(set(forced))
    if len(forced) > top_k:
        raise ValueError("more forced pages than top_k")
    fs = set(forced)
    rest = [p for p in range(len(scores)) if p not in fs]
    ranked = sorted(rest, key=lambda p: (-scores[p], p))
    return sorted(forced + ranked[:max(0, top_k - len(forced))])


def quest_decode_head(qs, keys, values, page_size: int, top_k: int, scale: float,
                      n_sink: int = 0, n_recent: int = 0, reduce: str = "sum"):
    """One (sequence, KV head) decode step after the newest token was appended.

    qs [G][D]: the query heads of the group; keys, values [L][D]: every
    resident token of this KV head in position order (L >= 1); n_sink,
    n_recent: pages always chosen; reduce: group aggregation of the bound.
    Returns dict(selected=list of pages, scores=[N_p], out=[G][D], lse=[G],
    tokens=array of token indices attended)."""
    qs = _f64(qs)
    keys = _f64(keys)
    values = _f64(values)
    L = keys.shape[0]
    mins, maxs = page_extrema(keys, page_size)
    scores = group_bound(qs, mins, maxs, reduce)
    selected = select_top_pages(scores, top_k, forced_pages(len(scores), n_sink, n_recent))
    tokens = np.concatenate([np.arange(p * page_size, min(L, (p + 1) * page_size))
                             for p in selected])
    G, D = qs.shape
    out = np.zeros((G, D))
    lse = np.zeros(G)
    for a in range(G):
        out[a], lse[a], _, _ = attend(qs[a], keys[tokens], values[tokens], scale)
    return dict(selected=selected, scores=scores, out=out, lse=lse, tokens=tokens,
                mins=mins, maxs=maxs)


def quest_decode(q, keys, values, lens, page_size: int, top_k: int, scale: float):
    """Batched form: q [B][H_q][D]; keys/values [B][H_kv][>=L_b][D]; lens [B].
    Returns (selected [B][H_kv][top_k] int with -1 padding, out [B][H_q][D],
    lse [B][H_q], scores list[B][H_kv] of arrays)."""
    q = _f64(q)
    B, Hq, D = q.shape
    Hkv = len(keys[0])
    G = Hq // Hkv
    sel = np.full((B, Hkv, top_k), -1, dtype=np.int64)
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    scores = [[None] * Hkv for _ in range(B)]
    for b in range(B):
        L = int(lens[b])
        for h in range(Hkv):
            r = quest_decode_head(q[b, h * G:(h + 1) * G], keys[b][h][:L], values[b][h][:L],
                                  page_size, top_k, scale)
            sel[b, h, :len(r["selected"])] = r["selected"]
            out[b, h * G:(h + 1) * G] = r["out"]
            lse[b, h * G:(h + 1) * G] = r["lse"]
            scores[b][h] = r["scores"]
    return sel, out, lse, scores
