"""Float64 CPU oracle of token-level sparse attention with a ReLU indexer
(DeepSeek Sparse Attention, DSA).

TEST INFRASTRUCTURE ONLY. Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The GPU
library never calls it and the two share no code: this file imports numpy
and nothing else.

What it computes, by source (the DSA how-to, bjdmk.com.cn/news/5181035):

* section 1: each query token interacts with only k key/value tokens
  (k = 2048), which takes the core attention from O(L^2) to O(L*k);
* section 3: a Lightning Indexer with 8 or 16 heads chooses those tokens; its
  linear layer, dot product and ReLU are its arithmetic (run in FP8 there),
  and it keeps one cached indexer key per token ("indexer key cache");
* section 4: for each query token the indexer picks top-k = 2048 key/value
  tokens and the attention then runs over them only (MLA in its absorbed
  form, where every query head reads one shared latent key/value);
* section 5: a top_k at or above the sequence length makes the sparse
  attention dense.

Readings taken where the page is silent (listed with reasons in the design
notes):

* D1  indexer score of key s for query t: I(t, s) = sum over indexer heads j
      of w[t, j] * ReLU(qi[t, j] . ki[s]); qi [Hi, Di] and the head weights
      w [Hi] are per query token, ki [Di] per key token (the cached indexer
      key), all given as inputs (the linear layers that make them from the
      hidden state are outside the attention step).
* D2  causal: the candidates of query t are the tokens s <= t. The chosen set
      is the top_k candidates by score, ties to the lower index; with t + 1 <=
      top_k every candidate is chosen. It is shared by all query heads of the
      token and exported ascending, padded with -1.
* D3  attention: each query head h attends with softmax scale 1/sqrt(D) over
      the chosen tokens of its KV head h // (Hq/G) (G = 1 is the absorbed
      MLA form: one key/value head for all query heads). No gate.
* D4  an injected selection is a set of tokens: entries outside [0, t] and
      repeats add nothing; a row with no usable entry gives an output of 0.
"""

from __future__ import annotations

import numpy as np


def indexer_scores(qi_t, ki, w_t) -> np.ndarray:
    """D1 for one query token: qi_t [Hi, Di], ki [N, Di], w_t [Hi] -> [N]."""
    qi_t = np.asarray(qi_t, dtype=np.float64)
    ki = np.asarray(ki, dtype=np.float64)
    w_t = np.asarray(w_t, dtype=np.float64)
    return (w_t[:, None] * np.maximum(qi_t @ ki.T, 0.0)).sum(axis=0)


def select_tokens(scores: np.ndarray, t: int, top_k: int):
    """D2: the top_k of candidates [0, t] (scores [t + 1]) by score, ties to
    the lower index. Returns (idx [top_k] int32 ascending, padded with -1;
    gap = the top_k-th largest score minus the (top_k + 1)-th, inf when every
    candidate is chosen)."""
    n = t + 1
    if n <= top_k:
        chosen = np.arange(n)
        gap = np.inf
    else:
        cand = np.asarray(scores[:n], dtype=np.float64)
        order = np.lexsort((np.arange(n), -cand))       # score descending, index ascending
        chosen = np.sort(order[:top_k])
        ranked = cand[order]
        gap = float(ranked[top_k - 1] - ranked[top_k])
    idx = np.full(top_k, -1, dtype=np.int32)
    idx[: len(chosen)] = chosen
    return idx, gap


def _attend(qh, keys, vals, scale):
    s = scale * (qh @ keys.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return (e / e.sum(axis=1, keepdims=True)) @ vals


def prefill(q, k, v, qi, ki, w, *, top_k: int, scale=None, rows=None, inject_idx=None,
            scores: bool = False) -> dict:
    """Token-level sparse attention over whole sequences.

    q [B, L, Hq, D]; k, v [B, L, G, D]; qi [B, L, Hi, Di]; ki [B, L, Di];
    w [B, L, Hi]; any float arrays holding the exact stored values. ``rows``
    restricts the query positions (all by default); ``inject_idx``
    [B, L, top_k] replaces the selection. Returns out [B, R, Hq, D],
    idx [B, R, top_k], gap [B, R] and, with ``scores``, the indexer scores
    [B, R, L] (NaN past each row's candidates).
    """
    B, L, Hq, D = q.shape
    G = k.shape[2]
    if Hq % G:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    Hg = Hq // G
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)
    res = {"out": np.zeros((B, R, Hq, D)), "idx": np.zeros((B, R, top_k), np.int32), "gap": np.zeros((B, R))}
    if scores:
        res["scores"] = np.full((B, R, L), np.nan)
    for b in range(B):
        K = np.asarray(k[b], dtype=np.float64)
        V = np.asarray(v[b], dtype=np.float64)
        KI = np.asarray(ki[b], dtype=np.float64)
        for r, t in enumerate(rows):
            t = int(t)
            if inject_idx is None:
                sc = indexer_scores(qi[b, t], KI[: t + 1], w[b, t])
                idx, gap = select_tokens(sc, t, top_k)
                if scores:
                    res["scores"][b, r, : t + 1] = sc
            else:
                idx, gap = np.asarray(inject_idx[b, t], dtype=np.int32), np.inf
            res["idx"][b, r], res["gap"][b, r] = idx, gap
            toks = sorted({int(j) for j in idx if 0 <= j <= t})     # D4
            if not toks:
                continue
            qt = np.asarray(q[b, t], dtype=np.float64)
            for g in range(G):
                hs = slice(g * Hg, (g + 1) * Hg)
                res["out"][b, r, hs] = _attend(qt[hs], K[toks, g], V[toks, g], scale)
    return res
