"""Pins of the token-level sparse attention oracle (oracle/dsa_ref.py), CPU only.

None re-types the oracle's formulas: each is a reduction to dense causal
attention (torch's scaled_dot_product_attention in float64), masked attention
over an explicit token mask (the same library routine), hand-built scores
whose top-k is known in advance, closed forms of the indexer written as loops,
or an invariant.
"""

import numpy as np
import pytest
import torch

from long_context_sparse_fwd_amd import inputs
from oracle import dsa_ref


def _data(L, Hq=4, G=1, D=16, Hi=4, Di=8, seed=0, batch=1):
    cfg = inputs.DsaConfig("t", batch, L, Hq, G, D, Hi, Di, "f32", top_k=8, seed=seed)
    raw = inputs.make_dsa_inputs(cfg, threads=1)
    return {k: inputs.to_f64(v, "f32") for k, v in raw.items()}


def _masked(q, k, v, allowed):
    """Attention of q [Hq, D] over the keys flagged in allowed [L] (k, v [L, G, D]),
    query head h reading KV head h // (Hq / G); torch SDPA in float64."""
    Hq, D = q.shape
    G = k.shape[1]
    kk = torch.from_numpy(np.repeat(k, Hq // G, axis=1).transpose(1, 0, 2).copy())[None]
    vv = torch.from_numpy(np.repeat(v, Hq // G, axis=1).transpose(1, 0, 2).copy())[None]
    qq = torch.from_numpy(q[:, None, :].copy())[None]
    mask = torch.from_numpy(np.asarray(allowed, dtype=bool))[None, None, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask,
                                                            scale=1.0 / np.sqrt(D))[0, :, 0].numpy()


@pytest.mark.parametrize("L,G", [(40, 1), (70, 2)])
def test_topk_at_or_above_length_is_dense_causal_attention(L, G):
    # top_k reaching the sequence length makes sparse attention dense: DSA
    # how-to (bjdmk.com.cn/news/5181035), section 5
    d = _data(L, Hq=4, G=G, seed=1)
    r = dsa_ref.prefill(d["q"], d["k"], d["v"], d["qi"], d["ki"], d["w"], top_k=L)
    Hq, D = 4, 16
    kk = torch.from_numpy(np.repeat(d["k"][0], Hq // G, axis=1).transpose(1, 0, 2).copy())[None]
    vv = torch.from_numpy(np.repeat(d["v"][0], Hq // G, axis=1).transpose(1, 0, 2).copy())[None]
    qq = torch.from_numpy(d["q"][0].transpose(1, 0, 2).copy())[None]
    dense = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True, scale=1 / np.sqrt(D))
    np.testing.assert_allclose(r["out"][0], dense[0].numpy().transpose(1, 0, 2), atol=1e-12)
    assert np.all(r["idx"][0, :, :] == np.where(np.arange(L)[None, :] <= np.arange(L)[:, None], np.arange(L), -1))


def test_indexer_score_by_explicit_loops():
    rng = np.random.default_rng(2)
    Hi, Di, N = 3, 5, 7
    qi, ki, w = rng.standard_normal((Hi, Di)), rng.standard_normal((N, Di)), rng.standard_normal(Hi)
    got = dsa_ref.indexer_scores(qi, ki, w)
    for s in range(N):
        acc = 0.0
        for j in range(Hi):
            dot = sum(qi[j, c] * ki[s, c] for c in range(Di))
            acc += w[j] * (dot if dot > 0 else 0.0)
        assert abs(got[s] - acc) < 1e-12


def test_selection_on_hand_built_scores_and_its_gap():
    sc = np.array([0.3, 0.9, -0.2, 0.9, 0.5, 0.1])
    idx, gap = dsa_ref.select_tokens(sc, 5, 3)
    assert list(idx) == [1, 3, 4] and abs(gap - (0.5 - 0.3)) < 1e-15      # ties of 0.9 both in
    idx, gap = dsa_ref.select_tokens(sc, 5, 1)
    assert list(idx) == [1] and gap == 0.0                                  # exact tie at the boundary: lower index
    idx, gap = dsa_ref.select_tokens(sc, 3, 2)                              # candidates 0..3 only (causal)
    assert list(idx) == [1, 3] and abs(gap - (0.9 - 0.3)) < 1e-15
    idx, gap = dsa_ref.select_tokens(sc, 2, 4)                              # fewer candidates than slots
    assert list(idx) == [0, 1, 2, -1] and np.isinf(gap)


def test_zero_head_weights_tie_everything_and_pick_the_lowest_tokens():
    L, k = 30, 6
    d = _data(L, seed=3)
    r = dsa_ref.prefill(d["q"], d["k"], d["v"], d["qi"], d["ki"], np.zeros_like(d["w"]), top_k=k, scores=True)
    for t in range(L):
        want = list(range(min(k, t + 1))) + [-1] * max(0, k - t - 1)
        assert list(r["idx"][0, t]) == want
    assert np.nanmax(np.abs(r["scores"])) == 0.0


def test_negative_weights_reverse_a_single_head_ranking():
    # one indexer head: score = w * ReLU(qi . ki); with w < 0 the chosen tokens
    # are those with the smallest positive dot products (zeros rank highest)
    L, k = 50, 5
    d = _data(L, Hi=1, seed=5)
    r = dsa_ref.prefill(d["q"], d["k"], d["v"], d["qi"], d["ki"], -np.abs(d["w"]), top_k=k)
    t = L - 1
    dots = np.array([float(d["qi"][0, t, 0] @ d["ki"][0, s]) for s in range(L)])
    relu = np.where(dots > 0, dots, 0.0)
    ranked = sorted(range(L), key=lambda s: (relu[s], s))          # ascending ReLU, then index
    assert list(r["idx"][0, t]) == sorted(ranked[:k])


def test_selection_is_the_top_of_a_full_sort_and_attention_is_masked_attention():
    L, k, G = 90, 12, 2
    d = _data(L, Hq=4, G=G, seed=7)
    r = dsa_ref.prefill(d["q"], d["k"], d["v"], d["qi"], d["ki"], d["w"], top_k=k, scores=True)
    for t in range(L):
        sc = r["scores"][0, t, : t + 1]
        desc = sorted(range(t + 1), key=lambda s: (-sc[s], s))
        chosen = sorted(desc[:k])
        assert list(r["idx"][0, t][: len(chosen)]) == chosen
        if t + 1 > k:
            assert abs(r["gap"][0, t] - (sc[desc[k - 1]] - sc[desc[k]])) < 1e-15
        allowed = np.zeros(L, bool)
        allowed[chosen] = True
        np.testing.assert_allclose(r["out"][0, t], _masked(d["q"][0, t], d["k"][0], d["v"][0], allowed), atol=1e-12)


def test_injected_selection_is_a_set_of_tokens():
    L, k = 40, 6
    d = _data(L, seed=9)
    rng = np.random.default_rng(4)
    inj = rng.integers(-3, L + 3, size=(1, L, k)).astype(np.int32)
    inj[0, :, 1] = inj[0, :, 0]
    inj[0, ::5] = -1
    r = dsa_ref.prefill(d["q"], d["k"], d["v"], d["qi"], d["ki"], d["w"], top_k=k, inject_idx=inj)
    for t in range(L):
        toks = {int(j) for j in inj[0, t] if 0 <= j <= t}
        if not toks:
            assert np.all(r["out"][0, t] == 0)
            continue
        allowed = np.array([s in toks for s in range(L)])
        np.testing.assert_allclose(r["out"][0, t], _masked(d["q"][0, t], d["k"][0], d["v"][0], allowed), atol=1e-12)


def test_output_is_linear_in_values_and_rows_option_matches_the_full_run():
    L, k = 45, 7
    d = _data(L, seed=11)
    r1 = dsa_ref.prefill(d["q"], d["k"], d["v"], d["qi"], d["ki"], d["w"], top_k=k)
    r2 = dsa_ref.prefill(d["q"], d["k"], -2.5 * d["v"], d["qi"], d["ki"], d["w"], top_k=k)
    np.testing.assert_allclose(r2["out"], -2.5 * r1["out"], atol=1e-12)
    r3 = dsa_ref.prefill(d["q"], d["k"], d["v"], d["qi"], d["ki"], d["w"], top_k=k, rows=[3, 44])
    np.testing.assert_allclose(r3["out"][0], r1["out"][0, [3, 44]], atol=0)
    np.testing.assert_array_equal(r3["idx"][0], r1["idx"][0, [3, 44]])


def test_prefill_scores_are_each_rows_own_indexer_scores():
    # the scores a row ranks come from that row's indexer query and head
    # weights against the keys up to it (explicit loops)
    L, Hi, Di = 20, 3, 8
    d = _data(L, Hi=Hi, Di=Di, seed=13)
    r = dsa_ref.prefill(d["q"], d["k"], d["v"], d["qi"], d["ki"], d["w"], top_k=4, rows=[0, 7, 19], scores=True)
    for i, t in enumerate([0, 7, 19]):
        for s in range(L):
            if s > t:
                assert np.isnan(r["scores"][0, i, s])
                continue
            acc = 0.0
            for j in range(Hi):
                dot = sum(d["qi"][0, t, j, c] * d["ki"][0, s, c] for c in range(Di))
                acc += d["w"][0, t, j] * max(dot, 0.0)
            assert abs(r["scores"][0, i, s] - acc) < 1e-12
