"""Pins of the oracle's general geometry (CPU only): a compression stride
below the block size (overlapping compressed blocks), selection blocks
larger than the compressed blocks, a learned compressor and a gate layer.

As for the plain geometry, none of these re-types the oracle's formulas:
each is a reduction to the plain geometry, a special case with a closed form,
a brute-force loop written independently on tiny inputs, a reformulation (the
selection-block scores as sums of a per-token mass), a library routine, or an
invariant.
"""

import numpy as np
import pytest
import torch

from oracle import nsa_ref
from tests.test_oracle import _data, _dense_causal


def _identity_mean_weights(block, D):
    w = np.zeros((D, block, D))
    for p in range(block):
        w[:, p, :] = np.eye(D) / block
    return w, np.zeros(D)


def test_general_entry_reduces_to_the_plain_geometry():
    # stride = block = select_block and a compressor whose weights take the
    # mean: the same outputs and selections as the plain block means
    L, Hq, G, D, l, n, w = 90, 4, 2, 8, 8, 3, 10
    d = _data(L, Hq, G, D, seed=51)
    plain = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=l, top_k=n, window=w, branches=True)
    wm, bm = _identity_mean_weights(l, D)
    gen = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=l, select_block=l, stride=l, top_k=n,
                          window=w, branches=True, cmp_weights=(wm, bm, wm, bm))
    np.testing.assert_array_equal(gen["idx"], plain["idx"])
    for key in ("out", "o_cmp", "o_slc", "o_win"):
        np.testing.assert_allclose(gen[key], plain[key], rtol=0, atol=1e-12)


def test_learned_compressor_by_explicit_loops():
    rng = np.random.default_rng(3)
    B, L, G, D, l, s = 2, 23, 2, 3, 5, 2
    x = rng.standard_normal((B, L, G, D))
    W = rng.standard_normal((D, l, D))
    bias = rng.standard_normal(D)
    got = nsa_ref.compress(x, l, s, W, bias)
    nc = 0
    while nc * s + l <= L:
        nc += 1
    assert got.shape == (B, nc, G, D)
    for b in range(B):
        for i in range(nc):
            for g in range(G):
                for o in range(D):
                    acc = bias[o]
                    for p in range(l):
                        for c in range(D):
                            acc += W[o, p, c] * x[b, i * s + p, g, c]
                    assert abs(got[b, i, g, o] - acc) < 1e-12


def test_overlapping_compressed_branch_is_masked_attention_over_explicit_block_means():
    L, Hq, G, D, l, s = 61, 4, 2, 8, 8, 3
    d = _data(L, Hq, G, D, seed=53)
    q, k, v = d["q"][0], d["k"][0], d["v"][0]
    starts = list(range(0, L - l + 1, s))               # blocks wholly inside the sequence
    kc = np.array([[k[a + i, g] for i in range(l)] for a in starts for g in range(G)]).reshape(
        len(starts), G, l, D).sum(axis=2) / l
    vc = np.array([[v[a + i, g] for i in range(l)] for a in starts for g in range(G)]).reshape(
        len(starts), G, l, D).sum(axis=2) / l
    ends = np.array([a + l - 1 for a in starts])
    Hg = Hq // G
    expect = np.zeros((L, Hq, D))
    for t in range(L):
        vis = ends <= t
        if not vis.any():
            continue
        for h in range(Hq):
            logits = np.where(vis, (kc[:, h // Hg] @ q[t, h]) / np.sqrt(D), -np.inf)
            p = np.exp(logits - logits.max())
            expect[t, h] = (p / p.sum()) @ vc[:, h // Hg]
    r = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=l, select_block=16, stride=s, top_k=2,
                        window=5, branches=True)
    np.testing.assert_allclose(r["o_cmp"][0], expect, rtol=0, atol=1e-12)
    assert np.all(r["o_cmp"][0, : l - 1] == 0)


@pytest.mark.parametrize("block,stride,select_block", [(8, 8, 16), (8, 4, 16), (8, 3, 8), (6, 4, 32), (8, 8, 8)])
def test_selection_scores_are_sums_of_a_token_mass(block, stride, select_block):
    # each compressed block's probability spread evenly over its tokens, then
    # summed per selection block
    rng = np.random.default_rng(block * 100 + stride * 10 + select_block)
    for t in (block - 1, 40, 97, 130):
        nvis = len(range(0, t - block + 2, stride))
        p = rng.uniform(size=nvis)
        own = t // select_block
        mass = np.zeros(t + 1)
        for i in range(nvis):
            mass[i * stride: i * stride + block] += p[i] / block
        want = np.array([mass[j * select_block: (j + 1) * select_block].sum() for j in range(own + 1)])
        got = nsa_ref.selection_scores(p, block, stride, select_block, own)
        # the plain geometry returns the visible blocks only: the rest carry no mass
        np.testing.assert_allclose(got, want[: len(got)], rtol=0, atol=1e-14)
        assert np.all(want[len(got):] == 0)
        assert abs(got.sum() - p.sum()) < 1e-12


def test_nested_selection_blocks_sum_their_compressed_blocks():
    # select_block = 2 * block, stride = block: each selection block holds
    # exactly two compressed blocks
    p = np.arange(1.0, 8.0)
    got = nsa_ref.selection_scores(p, 8, 8, 16, own=4)
    np.testing.assert_allclose(got, [1 + 2, 3 + 4, 5 + 6, 7, 0], atol=1e-15)


@pytest.mark.parametrize("L,block,stride,select_block", [(70, 8, 4, 16), (67, 4, 4, 8)])
def test_large_selection_blocks_are_dense_when_topk_covers_them(L, block, stride, select_block):
    d = _data(L, 4, 2, 16, seed=57)
    nsel = -(-L // select_block)
    r = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=block, select_block=select_block, stride=stride,
                        top_k=nsel, window=4, branches=True)
    dense = _dense_causal(d["q"][0], d["k"][0], d["v"][0])
    np.testing.assert_allclose(r["o_slc"][0], dense, rtol=0, atol=1e-12)


def test_general_selection_matches_brute_force_sort_and_score_mass():
    L, Hq, G, D, l, s, ls, n = 150, 6, 2, 8, 8, 4, 16, 4
    d = _data(L, Hq, G, D, seed=59)
    r = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=l, select_block=ls, stride=s, top_k=n, window=7,
                        scores=True, branches=True)
    for t in range(L):
        own = t // ls
        for g in range(G):
            sc = r["scores"][0, t, g]
            if t >= l - 1:
                assert abs(np.nansum(sc) - Hq // G) < 1e-12      # all probability mass lands in blocks 0..own
            idx = [int(j) for j in r["idx"][0, t, g] if j >= 0]
            assert own in idx and len(idx) == min(n, own + 1) and idx == sorted(idx)
            ranked = sorted(range(own), key=lambda j: (-sc[j], j))
            assert sorted(ranked[: n - 1] + [own]) == idx
            # the selected branch attends to the chosen selection blocks' tokens up to t
            toks = [x for j in idx for x in range(j * ls, min(j * ls + ls, t + 1))]
            hs = slice(g * (Hq // G), (g + 1) * (Hq // G))
            lg = (d["q"][0, t, hs] @ d["k"][0, toks, g].T) / np.sqrt(D)
            pr = np.exp(lg - lg.max(axis=1, keepdims=True))
            want = (pr / pr.sum(axis=1, keepdims=True)) @ d["v"][0, toks, g]
            np.testing.assert_allclose(r["o_slc"][0, t, hs], want, atol=1e-12)


def test_gate_layer_closed_form_and_library_routine():
    rng = np.random.default_rng(61)
    B, L, Hq, D = 2, 9, 3, 8
    q = rng.standard_normal((B, L, Hq, D))
    bias = rng.standard_normal((Hq, 3))
    g0 = nsa_ref.gates_from_query(q, np.zeros((Hq, D, 3)), bias)
    np.testing.assert_allclose(g0, np.broadcast_to(1 / (1 + np.exp(-bias)), g0.shape), atol=1e-15)
    W = rng.standard_normal((Hq, D, 3))
    want = torch.sigmoid(torch.einsum("blhd,hdc->blhc", torch.from_numpy(q), torch.from_numpy(W))
                         + torch.from_numpy(bias)).numpy()
    np.testing.assert_allclose(nsa_ref.gates_from_query(q, W, bias), want, atol=1e-14)


def test_general_decode_equals_prefill_row():
    L, Hq, G, D, l, s, ls, n, w = 100, 4, 2, 8, 8, 4, 16, 3, 10
    d = _data(L, Hq, G, D, seed=63, batch=2)
    rng = np.random.default_rng(2)
    wk, wv = rng.standard_normal((D, l, D)) / l, rng.standard_normal((D, l, D)) / l
    bk, bv = rng.standard_normal(D), rng.standard_normal(D)
    lens = np.array([L, 61])
    kcache = d["k"].transpose(0, 2, 1, 3).copy()
    vcache = d["v"].transpose(0, 2, 1, 3).copy()
    kc = nsa_ref.compress(d["k"], l, s, wk, bk).transpose(0, 2, 1, 3)
    vc = nsa_ref.compress(d["v"], l, s, wv, bv).transpose(0, 2, 1, 3)
    qd = np.stack([d["q"][b, lens[b] - 1] for b in range(2)])
    gd = np.stack([d["gates"][b, lens[b] - 1] for b in range(2)])
    rd = nsa_ref.decode(qd, kcache, vcache, kc, vc, lens, gd, block=l, select_block=ls, stride=s, top_k=n, window=w)
    for b in range(2):
        rp = nsa_ref.prefill(d["q"][b:b + 1], d["k"][b:b + 1], d["v"][b:b + 1], d["gates"][b:b + 1], block=l,
                             select_block=ls, stride=s, top_k=n, window=w, rows=[lens[b] - 1],
                             cmp_weights=(wk, bk, wv, bv))
        np.testing.assert_allclose(rd["out"][b], rp["out"][0, 0], atol=1e-13)
        np.testing.assert_array_equal(rd["idx"][b], rp["idx"][0, 0])
