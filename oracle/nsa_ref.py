"""Float64 CPU oracle of the Native Sparse Attention (NSA) forward pass.

TEST INFRASTRUCTURE ONLY. Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The GPU
library never calls it, and the two share no code: this file imports numpy and
nothing else.

It is deliberately plain and slow: one query position at a time, each step
written as its definition, all arithmetic in float64 on the exact stored input
values.

What it computes, by source (pages cited by title and section):

* NSA splits attention into three parallel branches -- a compressed branch for
  coarse global context, a selected branch that keeps fine-grained key blocks,
  and a sliding-window branch for local context -- whose outputs are merged by a
  gate: NSA how-to (qwbw.cn/news/106443), section 1.
* The parameters ``compress_block_size``, ``select_block_size``,
  ``select_top_k`` and ``sliding_window``: same page, section 3 (the
  ``[model.nsa]`` table of the config.toml skeleton).
* The selection dataflow -- compress each key block to one representation,
  score the blocks against the query, keep the top-k blocks, gather their
  tokens and attend over them; the choice depends on the query's content:
  NSA factory write-up (chencunli.com, "DeepSeek NSA on the Siemens 840D
  manual"), section "What dynamic sparsity actually sparsifies".

Readings taken where the pages are silent (the full list, with reasons, is in
the design notes):

* R1  compression is the arithmetic mean of each non-overlapping block of
      ``l`` tokens (stride ``l``); no learned weights exist here.
* R2  compressed block ``j`` is visible to query ``t`` only when the whole block
      is in the past: ``j*l + l - 1 <= t``. No visible block -> the compressed
      branch contributes 0 (its log-sum-exp is -inf).
* R3  block score = compressed-attention probability summed over the query
      heads of one KV group; the selection is shared by the group.
* R4  ``select_top_k`` counts the query's own block ``t // l``, which is always
      selected; the other ``n - 1`` are the best-scoring earlier blocks, ties to
      the lower index. Fewer candidates -> all of them, padded with -1.
* R5  the selected branch attends to the tokens of the chosen blocks that are
      at or before ``t``; the window branch to ``[max(0, t-w+1), t]``.
* R6  softmax scale ``1/sqrt(D)`` in all three branches; gates are given
      post-sigmoid values, one per (token, head, branch), not renormalised.
* R7  query head ``h`` belongs to KV group ``h // (Hq/G)``.
* R12 an injected selection is a set of blocks: entries outside ``[0, t//l]``
      and repeats add nothing; a row with no usable entry gives a selected
      branch of 0.

General geometry (the ``[model.nsa]`` table lists ``compress_block_size`` and
``select_block_size`` as separate fields; the factory write-up's sketch
compresses each block with a learned linear map of the flattened block):

* R14 compressed block ``i`` summarises tokens ``[i*d, i*d + l)`` for a
      compression stride ``1 <= d <= l`` (``d < l``: overlapping blocks); it
      exists when the whole block lies inside the sequence and is visible to
      query ``t`` when ``i*d + l - 1 <= t``. The summary is the block mean, or
      a linear map ``W[o, p, i]`` (output dim, position in the block, input
      dim) of the flattened block plus a bias ``b[o]``.
* R15 selection blocks hold ``l' >= l`` tokens: block ``j`` is
      ``[j*l', j*l' + l')``, the own block is ``t // l'``. A selection
      block's score is the compressed-attention mass on its tokens, each
      compressed block's probability spread evenly over the ``l`` tokens it
      summarises (with ``d = l = l'`` each compressed block is exactly one
      selection block and this is R3).
* R16 gates may come from a gate layer: ``gate[t, h, c] = sigmoid(q[t, h] .
      Wg[h, :, c] + bg[h, c])`` for the branches ``c`` in the order
      (compressed, selected, window); a one-layer MLP on the query, with
      synthetic weights here.
"""

from __future__ import annotations

import numpy as np


def n_compressed(L: int, block: int, stride: int) -> int:
    """Compressed blocks of an L-token sequence (R14): those wholly inside it."""
    return (L - block) // stride + 1 if L >= block else 0


def compress(x, block: int, stride=None, weight=None, bias=None) -> np.ndarray:
    """Compressed block representations: x [B, L, G, D] -> [B, Nc, G, D], float64.

    Stride ``block`` and no weight: the block means of R1 (a trailing partial
    block has no entry). Otherwise R14: block i covers tokens
    [i*stride, i*stride + block); its representation is the mean, or
    ``weight`` [D, block, D] (output dim, position, input dim) applied to the
    flattened block plus ``bias`` [D].
    """
    x = np.asarray(x, dtype=np.float64)
    B, L, G, D = x.shape
    if (stride is None or stride == block) and weight is None:
        nc = L // block
        return x[:, : nc * block].reshape(B, nc, block, G, D).mean(axis=2)
    stride = block if stride is None else stride
    nc = n_compressed(L, block, stride)
    out = np.zeros((B, nc, G, D))
    for i in range(nc):
        blk = x[:, i * stride: i * stride + block]          # [B, block, G, D]
        if weight is None:
            out[:, i] = blk.mean(axis=1)
        else:
            w = np.asarray(weight, dtype=np.float64)
            out[:, i] = np.einsum("opc,bpgc->bgo", w, blk) + np.asarray(bias, dtype=np.float64)
    return out


def selection_scores(cmp_scores: np.ndarray, block: int, stride: int, select_block: int, own: int) -> np.ndarray:
    """Selection-block scores from compressed-block scores (R15).

    ``cmp_scores`` [nvis] holds the scores of the visible compressed blocks.
    With stride == block == select_block they are the selection scores
    themselves; otherwise the result [own + 1] gives, for selection block j,
    the sum over compressed blocks i of score_i times the fraction of block
    i's tokens that lie in selection block j.
    """
    if stride == block == select_block:
        return cmp_scores
    out = np.zeros(own + 1)
    for i, si in enumerate(cmp_scores):
        lo, hi = i * stride, i * stride + block
        for j in range(lo // select_block, (hi - 1) // select_block + 1):
            overlap = min(hi, (j + 1) * select_block) - max(lo, j * select_block)
            out[j] += si * overlap / block
    return out


def gates_from_query(q, weight, bias) -> np.ndarray:
    """Gate layer (R16): q [B, L, Hq, D], weight [Hq, D, 3], bias [Hq, 3] ->
    gates [B, L, Hq, 3] = sigmoid(q . weight + bias), float64."""
    q = np.asarray(q, dtype=np.float64)
    z = np.einsum("blhd,hdc->blhc", q, np.asarray(weight, dtype=np.float64)) + np.asarray(bias, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def softmax_attend(qh: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float):
    """Plain softmax attention of ``qh`` [H, D] over ``keys``/``vals`` [N, D], N >= 1.

    Returns (out [H, D], lse [H]) with lse the natural-log normaliser of the
    scaled logits.
    """
    if keys.shape[0] == 0:
        raise ValueError("attention over an empty key set")
    s = scale * (qh @ keys.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return (e / z) @ vals, (m + np.log(z))[:, 0]


def select_blocks(scores: np.ndarray, own: int, top_k: int):
    """Selection rule R4 for one (query position, KV group).

    ``scores`` holds the block scores of every visible block; candidates are the
    blocks before the own block. Returns (idx [top_k] int32 ascending, padded
    with -1; gap) where gap is the (top_k-1)-th largest candidate score minus
    the top_k-th largest: the last chosen candidate against the first one
    left out. gap is inf when no score decides the set: every candidate is
    taken, or top_k == 1 (the own block alone, no candidate is chosen).
    """
    if own <= top_k - 1:
        chosen = list(range(own + 1))
        gap = np.inf
    else:
        cand = scores[:own]
        # primary key: score descending; secondary: block index ascending
        order = np.lexsort((np.arange(own), -cand))
        chosen = sorted(int(j) for j in order[: top_k - 1]) + [own]
        chosen.sort()
        ranked = cand[order]
        gap = float(ranked[top_k - 2] - ranked[top_k - 1]) if top_k >= 2 else np.inf
    idx = np.full(top_k, -1, dtype=np.int32)
    idx[: len(chosen)] = chosen
    return idx, gap


def nsa_token(q_t, K, V, Kc, Vc, t: int, g_t, *, block: int, top_k: int, window: int,
              scale: float, inject=None, select_block=None, stride=None) -> dict:
    """NSA forward for one query position ``t`` of one sequence.

    q_t [Hq, D]; K, V [T, G, D] with T > t (rows after t are never read);
    Kc, Vc [nc, G, D] holding at least the compressed blocks visible at t;
    g_t [Hq, 3] gates in the order (compressed, selected, window); inject
    [G, top_k] replaces the selection. ``select_block`` (l') and ``stride``
    (d) default to ``block`` (l).
    """
    q_t = np.asarray(q_t, dtype=np.float64)
    g_t = np.asarray(g_t, dtype=np.float64)
    Hq, D = q_t.shape
    G = K.shape[1]
    Hg = Hq // G
    d = block if stride is None else stride
    ls = block if select_block is None else select_block
    nvis = (t - block + 1) // d + 1 if t >= block - 1 else 0   # R2, R14
    own = t // ls                                           # R4, R15

    o_cmp = np.zeros((Hq, D))
    o_slc = np.zeros((Hq, D))
    o_win = np.zeros((Hq, D))
    lse = np.full(Hq, -np.inf)
    lse_slc = np.full(Hq, -np.inf)
    idx = np.full((G, top_k), -1, dtype=np.int32)
    gap = np.full(G, np.inf)
    group_scores = []

    for g in range(G):
        hs = slice(g * Hg, (g + 1) * Hg)      # R7
        qg = q_t[hs]
        # compressed branch over the visible block means
        if nvis > 0:
            kc = np.asarray(Kc[:nvis, g], dtype=np.float64)
            vc = np.asarray(Vc[:nvis, g], dtype=np.float64)
            o_cmp[hs], lse[hs] = softmax_attend(qg, kc, vc, scale)
            probs = np.exp(scale * (qg @ kc.T) - lse[hs][:, None])
            scores = probs.sum(axis=0)        # R3
        else:
            scores = np.zeros(0)
        scores = selection_scores(scores, block, d, ls, own)   # R15
        group_scores.append(scores)
        # block selection shared by the group
        if inject is None:
            idx[g], gap[g] = select_blocks(scores, own, top_k)
        else:
            idx[g] = np.asarray(inject[g], dtype=np.int32)
        # selected branch: tokens of the chosen blocks, causal (R5). The
        # selection is a set of blocks: repeated or unusable injected entries
        # add nothing, and no usable block leaves this branch at 0 (R12).
        blocks = sorted({int(j) for j in idx[g] if 0 <= j and j * ls <= t})
        if blocks:
            toks = np.concatenate([np.arange(j * ls, min(j * ls + ls, t + 1)) for j in blocks])
            o_slc[hs], lse_slc[hs] = softmax_attend(qg, np.asarray(K[toks, g], dtype=np.float64),
                                                    np.asarray(V[toks, g], dtype=np.float64), scale)
        # sliding-window branch (R5)
        lo = max(0, t - window + 1)
        o_win[hs], _ = softmax_attend(qg, np.asarray(K[lo: t + 1, g], dtype=np.float64),
                                      np.asarray(V[lo: t + 1, g], dtype=np.float64), scale)

    out = g_t[:, 0:1] * o_cmp + g_t[:, 1:2] * o_slc + g_t[:, 2:3] * o_win   # R6
    return {"out": out, "idx": idx, "lse": lse, "gap": gap, "lse_slc": lse_slc,
            "o_cmp": o_cmp, "o_slc": o_slc, "o_win": o_win, "scores": group_scores}


def _geometry(block: int, select_block, stride):
    """(l', d) with the defaults l' = d = l; 1 <= d <= l <= l' (R14, R15)."""
    ls = block if select_block is None else int(select_block)
    d = block if stride is None else int(stride)
    if not (1 <= d <= block <= ls):
        raise ValueError(f"need 1 <= stride ({d}) <= block ({block}) <= select_block ({ls})")
    return ls, d


def prefill(q, k, v, gates, *, block: int = 64, select_block=None, top_k: int, window: int,
            scale=None, inject_idx=None, rows=None, branches: bool = False,
            scores: bool = False, stride=None, cmp_weights=None) -> dict:
    """NSA prefill: every query position attends causally within its sequence.

    q [B, L, Hq, D]; k, v [B, L, G, D]; gates [B, L, Hq, 3]; any float dtype
    holding the exact stored values. ``rows`` restricts the output to the given
    query positions (all positions by default); K/V always span the full
    sequence. ``inject_idx`` [B, L, G, top_k] replaces the selection.
    ``select_block`` (l'), ``stride`` (d) and ``cmp_weights`` (wk, bk, wv, bv:
    the learned compressor of R14; None = block means) give the general
    geometry. Returns out [B, R, Hq, D], idx [B, R, G, top_k], lse [B, R, Hq]
    and gap [B, R, G] (plus the three branch outputs and the selected
    branch's own log-sum-exp ``lse_slc`` [B, R, Hq] when ``branches``, and
    the selection-block scores [B, R, G, ceil(L / l')] when ``scores``, NaN
    where undefined).
    """
    ls, d = _geometry(block, select_block, stride)
    B, L, Hq, D = q.shape
    G = k.shape[2]
    if Hq % G:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)
    res = {"out": np.zeros((B, R, Hq, D)), "idx": np.zeros((B, R, G, top_k), np.int32),
           "lse": np.zeros((B, R, Hq)), "gap": np.zeros((B, R, G))}
    if branches:
        for name in ("o_cmp", "o_slc", "o_win"):
            res[name] = np.zeros((B, R, Hq, D))
        res["lse_slc"] = np.zeros((B, R, Hq))
    fixed = list(res)
    if scores:
        res["scores"] = np.full((B, R, G, -(-L // ls)), np.nan)
    wk, bk, wv, bv = (None,) * 4 if cmp_weights is None else cmp_weights
    for b in range(B):
        K = np.asarray(k[b], dtype=np.float64)
        V = np.asarray(v[b], dtype=np.float64)
        Kc = compress(K[None], block, d, wk, bk)[0]
        Vc = compress(V[None], block, d, wv, bv)[0]
        for r, t in enumerate(rows):
            t = int(t)
            inj = None if inject_idx is None else inject_idx[b, t]
            one = nsa_token(q[b, t], K, V, Kc, Vc, t, gates[b, t], block=block, top_k=top_k,
                            window=window, scale=scale, inject=inj, select_block=ls, stride=d)
            for name in fixed:
                res[name][b, r] = one[name]
            if scores:
                for g, sg in enumerate(one["scores"]):
                    res["scores"][b, r, g, : len(sg)] = sg
    return res


def decode(q, k_cache, v_cache, kc_cache, vc_cache, seqlens, gates, *, block: int = 64,
           select_block=None, top_k: int, window: int, scale=None, inject_idx=None,
           branches: bool = False, stride=None) -> dict:
    """NSA decode: one new query per sequence at position ``seqlens[b] - 1``.

    q [B, Hq, D]; k_cache, v_cache [B, G, Lmax, D] already holding the new
    token; kc_cache, vc_cache [B, G, Nmax, D] holding the representations of
    the compressed blocks that lie wholly in the sequence (used as given);
    seqlens [B]; gates [B, Hq, 3]. Returns out [B, Hq, D], idx [B, G, top_k],
    lse [B, Hq], gap [B, G] and the selection-block scores
    [B, G, max(Nmax, ceil(Lmax / l'))] (NaN where undefined).
    """
    ls, d = _geometry(block, select_block, stride)
    B, Hq, D = q.shape
    G = k_cache.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    res = {"out": np.zeros((B, Hq, D)), "idx": np.zeros((B, G, top_k), np.int32),
           "lse": np.zeros((B, Hq)), "gap": np.zeros((B, G))}
    if branches:
        for name in ("o_cmp", "o_slc", "o_win"):
            res[name] = np.zeros((B, Hq, D))
    fixed = list(res)
    res["scores"] = np.full((B, G, max(kc_cache.shape[2], -(-k_cache.shape[2] // ls))), np.nan)
    for b in range(B):
        t = int(seqlens[b]) - 1
        nvis = n_compressed(t + 1, block, d)
        K = np.asarray(k_cache[b, :, : t + 1], dtype=np.float64).transpose(1, 0, 2)
        V = np.asarray(v_cache[b, :, : t + 1], dtype=np.float64).transpose(1, 0, 2)
        Kc = np.asarray(kc_cache[b, :, :nvis], dtype=np.float64).transpose(1, 0, 2)
        Vc = np.asarray(vc_cache[b, :, :nvis], dtype=np.float64).transpose(1, 0, 2)
        inj = None if inject_idx is None else inject_idx[b]
        one = nsa_token(q[b], K, V, Kc, Vc, t, gates[b], block=block, top_k=top_k,
                        window=window, scale=scale, inject=inj, select_block=ls, stride=d)
        for name in fixed:
            res[name][b] = one[name]
        for g, sg in enumerate(one["scores"]):
            res["scores"][b, g, : len(sg)] = sg
    return res
