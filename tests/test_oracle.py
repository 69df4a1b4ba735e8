"""Pins of the float64 oracle against facts fixed by the pages and by mathematics.

None of these re-types the oracle's own formulas. Each check is one of:
a special case that reduces to a textbook routine (dense causal attention via
torch's scaled_dot_product_attention in float64), a closed form, an invariant,
brute force on tiny inputs, or a planted input whose answer is known in
advance. Chosen so that a dropped branch, a wrong sign, an off-by-one in a mask
or a window, a transposed operand or a wrong head-to-group map each fails at
least one test.
"""

import numpy as np
import pytest
import torch

from long_context_sparse_fwd_amd import inputs
from oracle import nsa_ref


def _data(L, Hq, G, D, seed=0, dtype="f32", batch=1):
    cfg = inputs.PrefillConfig("t", batch, L, Hq, G, D, dtype, top_k=4, window=16, seed=seed)
    raw = inputs.make_prefill_inputs(cfg, threads=1)
    return {k: inputs.to_f64(v, dtype) for k, v in raw.items()}


def _dense_causal(q, k, v, lo_hi=None):
    """Dense causal attention per head with torch's SDPA in float64.

    q [L, Hq, D], k/v [L, G, D]; query head h reads KV head h // (Hq/G)."""
    L, Hq, D = q.shape
    G = k.shape[1]
    Hg = Hq // G
    kk = np.repeat(k, Hg, axis=1)
    vv = np.repeat(v, Hg, axis=1)
    qt = torch.from_numpy(q.transpose(1, 0, 2).copy())[None]
    kt = torch.from_numpy(kk.transpose(1, 0, 2).copy())[None]
    vt = torch.from_numpy(vv.transpose(1, 0, 2).copy())[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                         scale=1.0 / np.sqrt(D))
    return o[0].numpy().transpose(1, 0, 2)


# ---------------------------------------------------------------- I1 / I2

@pytest.mark.parametrize("L,block", [(40, 8), (67, 8), (130, 16)])
def test_selected_branch_is_dense_when_topk_covers_all_blocks(L, block):
    # top_k >= number of blocks makes the sparse selection dense: DSA how-to
    # (bjdmk.com.cn/news/5181035), section 5, on top_k reaching the length.
    d = _data(L, 4, 2, 16)
    nb = -(-L // block)
    r = nsa_ref.prefill(d["q"][..., :], d["k"], d["v"], d["gates"], block=block, top_k=nb,
                        window=4, branches=True)
    dense = _dense_causal(d["q"][0], d["k"][0], d["v"][0])
    np.testing.assert_allclose(r["o_slc"][0], dense, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,w", [(50, 50), (50, 400)])
def test_window_branch_is_dense_when_window_covers_sequence(L, w):
    d = _data(L, 4, 1, 8, seed=3)
    r = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=8, top_k=2, window=w,
                        branches=True)
    dense = _dense_causal(d["q"][0], d["k"][0], d["v"][0])
    np.testing.assert_allclose(r["o_win"][0], dense, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- I3

def test_compressed_branch_is_masked_attention_over_block_means():
    L, Hq, G, D, l = 70, 4, 2, 8, 8
    d = _data(L, Hq, G, D, seed=5)
    q, k, v = d["q"][0], d["k"][0], d["v"][0]
    nc = L // l
    # block means by explicit summation loops
    kc = np.zeros((nc, G, D))
    vc = np.zeros((nc, G, D))
    for j in range(nc):
        for i in range(l):
            kc[j] += k[j * l + i]
            vc[j] += v[j * l + i]
    kc /= l
    vc /= l
    # full logit matrix + explicit visibility mask, rows without a visible block -> 0
    t_idx = np.arange(L)[:, None]
    j_idx = np.arange(nc)[None, :]
    mask = (j_idx * l + l - 1) <= t_idx
    expect = np.zeros((L, Hq, D))
    Hg = Hq // G
    for h in range(Hq):
        logits = (q[:, h] @ kc[:, h // Hg].T) / np.sqrt(D)
        logits = np.where(mask, logits, -np.inf)
        for t in range(L):
            if not mask[t].any():
                continue
            p = np.exp(logits[t] - logits[t].max())
            p /= p.sum()
            expect[t, h] = p @ vc[:, h // Hg]
    r = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=l, top_k=3, window=5,
                        branches=True)
    np.testing.assert_allclose(r["o_cmp"][0], expect, rtol=0, atol=1e-12)
    # no visible block before t = l-1
    assert np.all(r["o_cmp"][0, : l - 1] == 0)
    assert np.all(np.isneginf(r["lse"][0, : l - 1]))


# ---------------------------------------------------------------- I4 / linearity

def test_one_hot_gates_isolate_each_branch_and_output_is_linear_in_gates():
    L, Hq, G, D = 48, 4, 2, 8
    d = _data(L, Hq, G, D, seed=7)
    base = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=8, top_k=3, window=6,
                           branches=True)
    for br, name in enumerate(["o_cmp", "o_slc", "o_win"]):
        gates = np.zeros_like(d["gates"])
        gates[..., br] = 1.0
        r = nsa_ref.prefill(d["q"], d["k"], d["v"], gates, block=8, top_k=3, window=6)
        np.testing.assert_allclose(r["out"], base[name], rtol=0, atol=1e-13)
    g1 = d["gates"]
    g2 = np.random.default_rng(1).uniform(size=g1.shape)
    r1 = nsa_ref.prefill(d["q"], d["k"], d["v"], g1, block=8, top_k=3, window=6)
    r2 = nsa_ref.prefill(d["q"], d["k"], d["v"], g2, block=8, top_k=3, window=6)
    r12 = nsa_ref.prefill(d["q"], d["k"], d["v"], g1 + 2.5 * g2, block=8, top_k=3, window=6)
    np.testing.assert_allclose(r12["out"], r1["out"] + 2.5 * r2["out"], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(r1["idx"], r2["idx"])


def test_output_is_linear_in_values():
    d = _data(40, 4, 1, 8, seed=9)
    r1 = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=8, top_k=2, window=5)
    r2 = nsa_ref.prefill(d["q"], d["k"], -3.0 * d["v"], d["gates"], block=8, top_k=2, window=5)
    np.testing.assert_allclose(r2["out"], -3.0 * r1["out"], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(r1["idx"], r2["idx"])


# ---------------------------------------------------------------- closed forms

def test_first_row_closed_form():
    # t = 0: no compressed block; the selected and window branches see only token 0.
    d = _data(20, 4, 2, 8, seed=11)
    r = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=8, top_k=3, window=4,
                        rows=[0])
    g = d["gates"][0, 0]
    v0 = d["v"][0, 0]
    expect = (g[:, 1:2] + g[:, 2:3]) * np.repeat(v0, 2, axis=0)
    np.testing.assert_allclose(r["out"][0, 0], expect, rtol=0, atol=1e-14)
    assert list(r["idx"][0, 0, 0]) == [0, -1, -1]


def test_row_l_minus_1_sees_exactly_block_zero():
    l, Hq, G, D = 8, 4, 2, 8
    d = _data(3 * l, Hq, G, D, seed=13)
    r = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=l, top_k=3, window=4,
                        rows=[l - 2, l - 1, 2 * l - 2], branches=True)
    # t = l-2: nothing visible; t = l-1 and t = 2l-2: only block 0, so the
    # compressed output is the plain mean of V over tokens 0..l-1
    assert np.all(r["o_cmp"][0, 0] == 0)
    vmean = d["v"][0, :l].sum(axis=0) / l
    for row in (1, 2):
        np.testing.assert_allclose(r["o_cmp"][0, row], np.repeat(vmean, 2, axis=0), atol=1e-14)
    one = nsa_ref.nsa_token(d["q"][0, l - 1], d["k"][0], d["v"][0],
                            nsa_ref.compress(d["k"], l)[0], nsa_ref.compress(d["v"], l)[0],
                            l - 1, d["gates"][0, l - 1], block=l, top_k=3, window=4,
                            scale=1 / np.sqrt(D))
    for s in one["scores"]:
        np.testing.assert_allclose(s, [Hq // G], atol=1e-14)


def test_zero_keys_give_plain_means_and_lowest_index_ties():
    # K = 0 makes every logit 0: each branch is a plain mean of its values, and
    # all block scores tie, so the tie rule picks the lowest block indices.
    L, Hq, G, D, l, n, w = 100, 4, 2, 8, 8, 4, 11
    d = _data(L, Hq, G, D, seed=17)
    k0 = np.zeros_like(d["k"])
    r = nsa_ref.prefill(d["q"], k0, d["v"], d["gates"], block=l, top_k=n, window=w,
                        branches=True)
    v = d["v"][0]
    for t in range(L):
        own, nvis = t // l, (t + 1) // l
        sel = list(range(min(own, n - 1))) + [own]
        toks = [i for j in sel for i in range(j * l, min(j * l + l, t + 1))]
        for g in range(G):
            assert list(r["idx"][0, t, g][: len(sel)]) == sel
            hs = slice(g * 2, g * 2 + 2)
            np.testing.assert_allclose(r["o_slc"][0, t, hs], np.broadcast_to(v[toks, g].mean(0), (2, D)),
                                       atol=1e-13)
            lo = max(0, t - w + 1)
            np.testing.assert_allclose(r["o_win"][0, t, hs],
                                       np.broadcast_to(v[lo: t + 1, g].mean(0), (2, D)), atol=1e-13)
            if nvis:
                np.testing.assert_allclose(r["o_cmp"][0, t, hs],
                                           np.broadcast_to(v[: nvis * l, g].mean(0), (2, D)), atol=1e-13)
        if own >= n:
            assert np.all(r["gap"][0, t] == 0)


def test_window_of_one_and_two():
    d = _data(30, 2, 1, 8, seed=19)
    q, k, v = d["q"][0], d["k"][0], d["v"][0]
    r1 = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=8, top_k=2, window=1,
                         branches=True)
    np.testing.assert_allclose(r1["o_win"][0], np.repeat(v, 2, axis=1), atol=1e-15)
    r2 = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=8, top_k=2, window=2,
                         branches=True)
    s = 1 / np.sqrt(8)
    for t in range(1, 30):
        for h in range(2):
            a = s * q[t, h] @ k[t - 1, 0]
            b = s * q[t, h] @ k[t, 0]
            expect = (np.exp(a) * v[t - 1, 0] + np.exp(b) * v[t, 0]) / (np.exp(a) + np.exp(b))
            np.testing.assert_allclose(r2["o_win"][0, t, h], expect, atol=1e-13)


def test_top1_is_own_block_attention():
    # with top_k = 1 only the own block is attended: dense causal attention
    # restricted to tokens [l*(t//l), t]
    L, l = 37, 8
    d = _data(L, 2, 1, 8, seed=23)
    r = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=l, top_k=1, window=3,
                        branches=True)
    for own in range(-(-L // l)):
        lo, hi = own * l, min(L, own * l + l)
        dense = _dense_causal(d["q"][0, lo:hi], d["k"][0, lo:hi], d["v"][0, lo:hi])
        np.testing.assert_allclose(r["o_slc"][0, lo:hi], dense, atol=1e-12)
        assert np.all(r["idx"][0, lo:hi, 0, 0] == own)


# ---------------------------------------------------------------- injected selections (R12)

def _masked_attention(q, k, v, allowed):
    """Attention of one query per head over the keys flagged in ``allowed`` [L],
    with torch's SDPA in float64. q [Hq, D], k/v [L, G, D]."""
    Hq, D = q.shape
    G = k.shape[1]
    Hg = Hq // G
    kk = torch.from_numpy(np.repeat(k, Hg, axis=1).transpose(1, 0, 2).copy())[None]
    vv = torch.from_numpy(np.repeat(v, Hg, axis=1).transpose(1, 0, 2).copy())[None]
    qq = torch.from_numpy(q[:, None, :].copy())[None]
    mask = torch.from_numpy(np.asarray(allowed, dtype=bool))[None, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=1.0 / np.sqrt(D))
    return o[0, :, 0].numpy()


def test_injected_selection_is_a_set_of_blocks():
    # repeats and unusable entries (negative, or later than the own block) add
    # nothing: the selected branch is attention over the union of the usable
    # blocks' tokens at or before t
    L, Hq, G, D, l, n = 50, 4, 2, 8, 8, 5
    d = _data(L, Hq, G, D, seed=31)
    rng = np.random.default_rng(5)
    inj = rng.integers(-2, L // l + 2, size=(1, L, G, n)).astype(np.int32)
    inj[0, :, :, 1] = inj[0, :, :, 0]            # a repeat in every row
    r = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=l, top_k=n, window=4,
                        inject_idx=inj, branches=True)
    Hg = Hq // G
    for t in range(L):
        for g in range(G):
            blocks = {int(j) for j in inj[0, t, g] if 0 <= j <= t // l}
            hs = slice(g * Hg, (g + 1) * Hg)
            if not blocks:
                assert np.all(r["o_slc"][0, t, hs] == 0.0)
                continue
            allowed = np.array([(key // l) in blocks and key <= t for key in range(L)])
            want = _masked_attention(d["q"][0, t, hs], d["k"][0][:, g:g + 1], d["v"][0][:, g:g + 1], allowed)
            np.testing.assert_allclose(r["o_slc"][0, t, hs], want, atol=1e-12)


def test_empty_injected_selection_drops_the_selected_branch():
    L, Hq, G, D, l, n = 24, 2, 1, 8, 8, 3
    d = _data(L, Hq, G, D, seed=37)
    inj = np.full((1, L, G, n), -1, dtype=np.int32)
    r = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=l, top_k=n, window=5,
                        inject_idx=inj, branches=True)
    assert np.all(r["o_slc"] == 0.0)
    gates = d["gates"]
    np.testing.assert_allclose(r["out"], gates[..., 0:1] * r["o_cmp"] + gates[..., 2:3] * r["o_win"],
                               atol=1e-14)


# ---------------------------------------------------------------- selection

def test_selection_matches_brute_force_sort_and_score_mass():
    L, Hq, G, D, l, n = 160, 6, 2, 8, 8, 5
    d = _data(L, Hq, G, D, seed=29)
    kc = nsa_ref.compress(d["k"], l)[0]
    vc = nsa_ref.compress(d["v"], l)[0]
    for t in range(L):
        one = nsa_ref.nsa_token(d["q"][0, t], d["k"][0], d["v"][0], kc, vc, t, d["gates"][0, t],
                                block=l, top_k=n, window=7, scale=1 / np.sqrt(D))
        own = t // l
        for g in range(G):
            s = one["scores"][g]
            if (t + 1) // l:
                assert abs(s.sum() - Hq // G) < 1e-12       # probabilities of Hg heads
            idx = [int(j) for j in one["idx"][g] if j >= 0]
            assert own in idx and len(idx) == min(n, own + 1)
            assert idx == sorted(idx)
            ranked = sorted(range(own), key=lambda j: (-s[j], j))
            assert sorted(ranked[: n - 1] + [own]) == idx


def test_planted_blocks_are_selected_per_group():
    # Group 0's heads look along +e0, group 1's along +e1; a few planted key
    # blocks point the same way and must be chosen, each only for its own group.
    L, Hq, G, D, l, n = 128, 4, 2, 8, 8, 4
    rng = np.random.default_rng(0)
    q = 0.01 * rng.standard_normal((1, L, Hq, D))
    k = 0.01 * rng.standard_normal((1, L, G, D))
    v = rng.standard_normal((1, L, G, D))
    q[0, :, 0:2, 0] += 4.0
    q[0, :, 2:4, 1] += 4.0
    plant = {0: [2, 5, 9], 1: [1, 7, 11]}
    for g, blocks in plant.items():
        for j in blocks:
            k[0, j * l:(j + 1) * l, g, g] += 4.0
            # a decoy along the other group's direction
            k[0, j * l:(j + 1) * l, 1 - g, 1 - g] -= 4.0
    gates = np.ones((1, L, Hq, 3))
    r = nsa_ref.prefill(q, k, v, gates, block=l, top_k=n, window=8, rows=[L - 1, 100])
    for row, t in enumerate([L - 1, 100]):
        own = t // l
        for g in range(G):
            assert list(r["idx"][0, row, g]) == sorted(plant[g] + [own])


# ---------------------------------------------------------------- prefix / decode

def test_causal_prefix_consistency():
    # The keyed generator makes a shorter workload a prefix of a longer one, and
    # causality makes the shorter run's outputs a prefix of the longer run's.
    a = _data(48, 4, 2, 8, seed=31)
    b = _data(80, 4, 2, 8, seed=31)
    np.testing.assert_array_equal(a["q"], b["q"][:, :48])
    ra = nsa_ref.prefill(a["q"], a["k"], a["v"], a["gates"], block=8, top_k=3, window=9)
    rb = nsa_ref.prefill(b["q"], b["k"], b["v"], b["gates"], block=8, top_k=3, window=9)
    np.testing.assert_allclose(ra["out"], rb["out"][:, :48], atol=1e-13)
    np.testing.assert_array_equal(ra["idx"], rb["idx"][:, :48])


def test_decode_equals_prefill_row():
    L, Hq, G, D, l, n, w = 90, 4, 2, 8, 8, 3, 10
    d = _data(L, Hq, G, D, seed=37, batch=2)
    lens = np.array([L, 57])
    B = 2
    kcache = d["k"].transpose(0, 2, 1, 3).copy()           # [B, G, L, D]
    vcache = d["v"].transpose(0, 2, 1, 3).copy()
    kc = nsa_ref.compress(d["k"], l).transpose(0, 2, 1, 3)  # [B, G, Nc, D]
    vc = nsa_ref.compress(d["v"], l).transpose(0, 2, 1, 3)
    qd = np.stack([d["q"][b, lens[b] - 1] for b in range(B)])
    gd = np.stack([d["gates"][b, lens[b] - 1] for b in range(B)])
    rd = nsa_ref.decode(qd, kcache, vcache, kc, vc, lens, gd, block=l, top_k=n, window=w)
    for b in range(B):
        rp = nsa_ref.prefill(d["q"][b:b + 1], d["k"][b:b + 1], d["v"][b:b + 1],
                             d["gates"][b:b + 1], block=l, top_k=n, window=w, rows=[lens[b] - 1])
        np.testing.assert_allclose(rd["out"][b], rp["out"][0, 0], atol=1e-13)
        np.testing.assert_array_equal(rd["idx"][b], rp["idx"][0, 0])


# ---------------------------------------------------------------- edge shapes

def test_edge_shapes():
    # shorter than one block: nothing compressed, only block 0 selectable
    d = _data(5, 2, 1, 8, seed=41)
    r = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=8, top_k=4, window=3,
                        branches=True)
    assert np.all(r["o_cmp"] == 0)
    assert np.all(r["idx"][0, :, 0] == np.array([0, -1, -1, -1]))
    dense = _dense_causal(d["q"][0], d["k"][0], d["v"][0])
    np.testing.assert_allclose(r["o_slc"][0], dense, atol=1e-13)
    # injected indices replace the selection
    inj = np.zeros((1, 5, 1, 4), np.int32) - 1
    inj[..., 0] = 0
    r2 = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=8, top_k=4, window=3,
                         inject_idx=inj)
    np.testing.assert_allclose(r2["out"], r["out"], atol=1e-15)
    # selection blocks smaller than the compressed blocks, or a stride past the block: rejected
    with pytest.raises(ValueError):
        nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=8, select_block=4, top_k=2, window=3)
    with pytest.raises(ValueError):
        nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=8, stride=9, top_k=2, window=3)


# ---------------------------------------------------------------- generator

def test_generator_bf16_rounding_matches_torch_rne():
    x = np.random.default_rng(3).standard_normal(100000).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]   # exact ties
    ours = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_generator_is_deterministic_and_prefix_stable():
    c1 = inputs.PrefillConfig("a", 1, 100, 4, 2, 8, "bf16", top_k=2, window=4)
    c2 = inputs.PrefillConfig("b", 1, 200, 4, 2, 8, "bf16", top_k=2, window=4)
    a, b = inputs.make_prefill_inputs(c1), inputs.make_prefill_inputs(c2)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key][:, :100])
    dc = inputs.DecodeConfig("d", 1, 200, 4, 2, 8, "bf16", top_k=2, window=4, seqlens=(150,))
    d = inputs.make_decode_inputs(dc)
    np.testing.assert_array_equal(d["q"][0], b["q"][0, 149])
    np.testing.assert_array_equal(d["k_cache"][0], b["k"][0].transpose(1, 0, 2))
    np.testing.assert_array_equal(d["gates"][0], b["gates"][0, 149])
    g = inputs.to_f64(b["gates"], "bf16")
    assert np.all((g > 0) & (g < 1))


# ---------------------------------------------------------------- selection gap

@pytest.mark.parametrize("top_k,idx,gap", [
    # candidates 0..4 score 0.5, 0.1, 0.9, 0.35, 0.62; the own block is 5
    (1, [5], np.inf),                      # own block alone: no score decides anything
    (2, [2, 5], 0.9 - 0.62),               # last chosen 0.9, first left out 0.62
    (3, [2, 4, 5], 0.62 - 0.5),
    (4, [0, 2, 4, 5], 0.5 - 0.35),
    (5, [0, 2, 3, 4, 5], 0.35 - 0.1),      # own == top_k: one candidate left out
    (6, [0, 1, 2, 3, 4, 5], np.inf),       # own == top_k - 1: every candidate taken
    (8, [0, 1, 2, 3, 4, 5, -1, -1], np.inf),
])
def test_selection_gap_on_hand_built_scores(top_k, idx, gap):
    # Check A's excuse rule reads this gap: the score of the last candidate the
    # rule keeps minus the score of the first one it leaves out.
    scores = np.array([0.5, 0.1, 0.9, 0.35, 0.62, 0.01])   # the last entry is the own block's
    got_idx, got_gap = nsa_ref.select_blocks(scores, 5, top_k)
    assert list(got_idx) == idx
    if np.isinf(gap):
        assert np.isinf(got_gap) and got_gap > 0
    else:
        assert abs(got_gap - gap) < 1e-15


def test_selection_gap_at_a_near_tie_and_an_exact_tie():
    # a 1e-9 lead decides the boundary: the gap is that lead
    idx, gap = nsa_ref.select_blocks(np.array([0.3, 0.3 + 1e-9, 0.1, 0.2]), 4, 2)
    assert list(idx) == [1, 4] and abs(gap - 1e-9) < 1e-15
    idx, gap = nsa_ref.select_blocks(np.array([0.3, 0.3 + 1e-9, 0.1, 0.2]), 4, 3)
    assert list(idx) == [0, 1, 4] and abs(gap - 0.1) < 1e-15
    # an exact tie at the boundary: the lower index wins and the gap is 0
    idx, gap = nsa_ref.select_blocks(np.array([0.2, 0.3, 0.3, 0.1]), 4, 2)
    assert list(idx) == [1, 4] and gap == 0.0


def test_prefill_gap_is_the_boundary_of_a_full_sort_of_its_scores():
    # through the whole prefill: for rows with own == top_k - 1 (all taken),
    # own == top_k (one left out) and own > top_k, the reported gap is the
    # difference between ranks top_k - 1 and top_k of a plain descending sort
    # of the row's candidate scores, and the chosen set is the top of that sort
    L, Hq, G, D, l, n = 120, 6, 2, 8, 8, 4
    d = _data(L, Hq, G, D, seed=43)
    rows = [3 * l, 3 * l + 5, 4 * l, 4 * l + 7, 10 * l, L - 1]
    r = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=l, top_k=n, window=6, rows=rows,
                        scores=True)
    for i, t in enumerate(rows):
        own = t // l
        for g in range(G):
            cand = [(float(r["scores"][0, i, g, j]), j) for j in range(own)]
            if own <= n - 1:
                assert np.isinf(r["gap"][0, i, g])
                continue
            desc = sorted(cand, key=lambda sj: (-sj[0], sj[1]))
            want = desc[n - 2][0] - desc[n - 1][0]
            assert abs(r["gap"][0, i, g] - want) < 1e-15
            assert r["gap"][0, i, g] > 0                       # distinct random scores
            assert sorted(j for _, j in desc[: n - 1]) + [own] == list(r["idx"][0, i, g])
