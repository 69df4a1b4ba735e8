"""Float64 CPU oracle of the Native Sparse Attention (NSA) backward pass.

TEST INFRASTRUCTURE ONLY. Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The GPU
library never calls it, and the two share no code: this file imports numpy and
the forward oracle next to it, nothing else.

The gradients of the prefill output with respect to q, k, v and the gates,
given the upstream gradient ``dout`` and a FIXED block selection (the top-k
choice is piecewise constant in its inputs, so it carries no gradient; the
selection is an input here, exactly as an injected selection is for the
forward). The pages present NSA as trained end to end with speedups claimed
for the backward pass as well (NSA how-to, qwbw.cn/news/106443, section 1);
they give no formulas for it, so this is the textbook gradient of the forward
the forward oracle defines:

* each branch x in (compressed, selected, window) is softmax attention of the
  query heads over its key set; with o_x its output, P its probabilities and
  dO_x = g_x * dout the gradient reaching it,
    dgate_x = dout . o_x,
    dS = P * (dO_x V^T - rowsum(dO_x * o_x)),
    dq += scale dS K,  dK_set += scale dS^T q,  dV_set += P^T dO_x;
* the compressed branch's keys and values are block means (reading R1), so
  its key/value gradients are spread evenly over the 64 tokens of each block.

Same readings as the forward oracle (R1-R12), same argument conventions.
Plain and slow: one query position and KV group at a time.
"""

from __future__ import annotations

import numpy as np

from .nsa_ref import compress


def _attend_backward(qg, keys, vals, dout_g, gate, scale):
    """Backward of softmax attention of qg [H, D] over keys/vals [N, D] (N >= 1).

    dout_g [H, D] is the gradient of the gated sum with respect to this
    branch's gated output; gate [H] the branch's gate. Returns
    (dgate [H], dq [H, D], dkeys [N, D], dvals [N, D]).
    """
    s = scale * (qg @ keys.T)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    o = p @ vals
    dgate = (dout_g * o).sum(axis=1)
    do = gate[:, None] * dout_g
    dp = do @ vals.T
    ds = p * (dp - (do * o).sum(axis=1, keepdims=True))
    return dgate, scale * (ds @ keys), scale * (ds.T @ qg), p.T @ do


def prefill_backward(q, k, v, gates, dout, idx, *, block: int = 64, select_block=None,
                     top_k: int, window: int, scale=None, rows=None) -> dict:
    """Gradients of the NSA prefill for a fixed selection ``idx`` [B, L, G, top_k].

    q [B, L, Hq, D]; k, v [B, L, G, D]; gates [B, L, Hq, 3]; dout [B, L, Hq, D].
    ``idx`` follows the injected-selection rule R12 (a set of blocks; entries
    outside [0, t // block] and repeats add nothing). Returns float64 dq, dk,
    dv and dgates of the input shapes. ``rows`` restricts the query positions
    taken into account (all by default): dq and dgates are then filled for
    those rows only, and dk / dv hold the sums over those rows' terms, which is
    the whole gradient for keys seen by no other row.
    """
    if select_block is not None and select_block != block:
        raise NotImplementedError("the backward oracle covers selection blocks equal to the compressed blocks")
    B, L, Hq, D = q.shape
    G = k.shape[2]
    Hg = Hq // G
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dq = np.zeros((B, L, Hq, D))
    dk = np.zeros((B, L, G, D))
    dv = np.zeros((B, L, G, D))
    dgates = np.zeros((B, L, Hq, 3))
    for b in range(B):
        K = np.asarray(k[b], dtype=np.float64)
        V = np.asarray(v[b], dtype=np.float64)
        Kc = compress(K[None], block)[0]
        Vc = compress(V[None], block)[0]
        dKc = np.zeros_like(Kc)
        dVc = np.zeros_like(Vc)
        for t in (range(L) if rows is None else rows):
            t = int(t)
            qt = np.asarray(q[b, t], dtype=np.float64)
            gt = np.asarray(gates[b, t], dtype=np.float64)
            dt = np.asarray(dout[b, t], dtype=np.float64)
            nvis = (t + 1) // block
            for g in range(G):
                hs = slice(g * Hg, (g + 1) * Hg)
                qg, dg, gg = qt[hs], dt[hs], gt[hs]
                # compressed branch: block means, whole blocks in the past (R2)
                if nvis > 0:
                    dgt, dqx, dkx, dvx = _attend_backward(qg, Kc[:nvis, g], Vc[:nvis, g], dg, gg[:, 0], scale)
                    dgates[b, t, hs, 0] = dgt
                    dq[b, t, hs] += dqx
                    dKc[:nvis, g] += dkx
                    dVc[:nvis, g] += dvx
                # selected branch over the set of usable blocks (R5, R12)
                blocks = sorted({int(j) for j in idx[b, t, g] if 0 <= j and j * block <= t})
                if blocks:
                    toks = np.concatenate([np.arange(j * block, min(j * block + block, t + 1)) for j in blocks])
                    dgt, dqx, dkx, dvx = _attend_backward(qg, K[toks, g], V[toks, g], dg, gg[:, 1], scale)
                    dgates[b, t, hs, 1] = dgt
                    dq[b, t, hs] += dqx
                    dk[b, toks, g] += dkx
                    dv[b, toks, g] += dvx
                # window branch (R5)
                lo = max(0, t - window + 1)
                dgt, dqx, dkx, dvx = _attend_backward(qg, K[lo: t + 1, g], V[lo: t + 1, g], dg, gg[:, 2], scale)
                dgates[b, t, hs, 2] = dgt
                dq[b, t, hs] += dqx
                dk[b, lo: t + 1, g] += dkx
                dv[b, lo: t + 1, g] += dvx
        # a block mean's gradient reaches each of its tokens divided by the block size (R1)
        nc = Kc.shape[0]
        dk[b, : nc * block] += np.repeat(dKc / block, block, axis=0)
        dv[b, : nc * block] += np.repeat(dVc / block, block, axis=0)
    return {"dq": dq, "dk": dk, "dv": dv, "dgates": dgates}
