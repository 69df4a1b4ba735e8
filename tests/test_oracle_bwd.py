"""Pins of the float64 backward oracle against facts independent of its formulas.

Each check is one of: central finite differences of the forward oracle (the
selection held fixed by injecting it), a special case that reduces to dense
causal attention differentiated by torch autograd in float64, or a closed form
that the gradients of softmax attention satisfy. A wrong sign, a dropped
rowsum term, a transposed operand, a missing 1/block in the block-mean
gradient or a wrong visibility mask each fails at least one of them.
"""

import numpy as np
import pytest
import torch

from long_context_sparse_fwd_amd import inputs
from oracle import nsa_bwd_ref, nsa_ref


def _data(L, Hq, G, D, seed=0, batch=1, top_k=3, window=20, block=16):
    cfg = inputs.PrefillConfig("t", batch, L, Hq, G, D, "f32", top_k=top_k, window=window, seed=seed)
    raw = inputs.make_prefill_inputs(cfg, threads=1)
    d = {k: inputs.to_f64(v, "f32") for k, v in raw.items()}
    d["dout"] = inputs.to_f64(inputs.make_dout(cfg), "f32")
    return d


def _loss(d, idx, block, top_k, window, **over):
    x = dict(d, **over)
    r = nsa_ref.prefill(x["q"], x["k"], x["v"], x["gates"], block=block, top_k=top_k, window=window,
                        inject_idx=idx)
    return float((r["out"] * d["dout"]).sum())


@pytest.mark.parametrize("seed,inject_odd", [(0, False), (5, True)])
def test_gradients_match_finite_differences(seed, inject_odd):
    # L = 70 with blocks of 16: a partial last block, 4 complete block means,
    # selections of up to 3 blocks, a window shorter than the sequence.
    block, top_k, window = 16, 3, 20
    d = _data(70, 4, 2, 8, seed=seed, top_k=top_k, window=window, block=block)
    idx = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=block, top_k=top_k,
                          window=window)["idx"]
    if inject_odd:  # repeats and unusable entries count as in the forward (a set of blocks)
        idx = idx.copy()
        idx[0, 40:50, 0, 2] = idx[0, 40:50, 0, 0]
        idx[0, 55:60, 1, 1] = 9
        idx[0, 60:62, 1, :] = -1
    g = nsa_bwd_ref.prefill_backward(d["q"], d["k"], d["v"], d["gates"], d["dout"], idx, block=block,
                                     top_k=top_k, window=window)
    rng = np.random.default_rng(seed)
    h = 1e-5
    for name, grad in (("q", g["dq"]), ("k", g["dk"]), ("v", g["dv"]), ("gates", g["dgates"])):
        x = d[name]
        for _ in range(12):
            pos = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[pos] += h
            xm[pos] -= h
            fd = (_loss(d, idx, block, top_k, window, **{name: xp}) -
                  _loss(d, idx, block, top_k, window, **{name: xm})) / (2 * h)
            assert abs(fd - grad[pos]) <= 1e-7 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])


def _torch_dense_grads(q, k, v, dout, gate_col, gates):
    """Causal attention per head (query head h reads KV head h // (Hq/G)),
    differentiated by torch autograd in float64; the output is scaled by the
    given gate column, as in the gated sum."""
    L, Hq, D = q.shape
    G = k.shape[1]
    Hg = Hq // G
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    kk = kt.repeat_interleave(Hg, dim=1).permute(1, 0, 2)[None]
    vv = vt.repeat_interleave(Hg, dim=1).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt.permute(1, 0, 2)[None], kk, vv, is_causal=True,
                                                         scale=1.0 / np.sqrt(D))[0].permute(1, 0, 2)
    gt = torch.tensor(gates[..., gate_col])[..., None]
    (o * gt * torch.tensor(dout)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy(), (o.detach().numpy() * dout).sum(-1)


@pytest.mark.parametrize("branch", ["window", "selected"])
def test_dense_special_cases_match_torch_autograd(branch):
    # Window covering the whole sequence, or a selection of every block up to
    # the own one: that branch is dense causal attention. The other two gates
    # are zero, so only its gradients remain.
    block, L = 16, 75
    d = _data(L, 4, 2, 8, seed=2)
    col = 2 if branch == "window" else 1
    gates = np.zeros_like(d["gates"])
    gates[..., col] = d["gates"][..., col]
    nb = -(-L // block)
    idx = np.tile(np.arange(nb, dtype=np.int32), (1, L, 2, 1))
    g = nsa_bwd_ref.prefill_backward(d["q"], d["k"], d["v"], gates, d["dout"], idx, block=block, top_k=nb,
                                     window=L if branch == "window" else 3)
    dq, dk, dv, dgate = _torch_dense_grads(d["q"][0], d["k"][0], d["v"][0], d["dout"][0], col, gates[0])
    for got, want in ((g["dq"][0], dq), (g["dk"][0], dk), (g["dv"][0], dv), (g["dgates"][0, ..., col], dgate)):
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-11)


def test_compressed_branch_matches_torch_autograd_through_block_means():
    # Gates (1, 0, 0): attention over the block means with whole blocks in
    # the past, written as a masked dense product in torch and differentiated
    # through the mean pooling by autograd (a row with no visible block
    # contributes nothing).
    block, L, Hq, G, D = 8, 45, 4, 2, 8
    d = _data(L, Hq, G, D, seed=4)
    gates = np.zeros_like(d["gates"])
    gates[..., 0] = d["gates"][..., 0]
    idx = np.full((1, L, G, 2), -1, np.int32)
    g = nsa_bwd_ref.prefill_backward(d["q"], d["k"], d["v"], gates, d["dout"], idx, block=block, top_k=2,
                                     window=4)
    qt = torch.tensor(d["q"][0], requires_grad=True)
    kt = torch.tensor(d["k"][0], requires_grad=True)
    vt = torch.tensor(d["v"][0], requires_grad=True)
    nc = L // block
    kc = kt[: nc * block].reshape(nc, block, G, D).mean(1).repeat_interleave(Hq // G, 1)  # [nc, Hq, D]
    vc = vt[: nc * block].reshape(nc, block, G, D).mean(1).repeat_interleave(Hq // G, 1)
    s = torch.einsum("thd,chd->htc", qt, kc) / np.sqrt(D)
    vis = torch.tensor(np.arange(nc)[None, :] * block + block - 1 <= np.arange(L)[:, None])  # [t, c]
    s = s.masked_fill(~vis[None], float("-inf"))
    p = torch.softmax(s, -1).nan_to_num(0.0)
    o = torch.einsum("htc,chd->thd", p, vc)
    (o * torch.tensor(gates[0, ..., 0:1]) * torch.tensor(d["dout"][0])).sum().backward()
    np.testing.assert_allclose(g["dq"][0], qt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dk"][0], kt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dv"][0], vt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dgates"][0, ..., 0], (o.detach().numpy() * d["dout"][0]).sum(-1),
                               rtol=0, atol=1e-11)


def test_closed_form_sums_of_key_and_value_gradients():
    # Adding one vector to every key of a group (and so to every block mean)
    # leaves each softmax unchanged: the key gradients of a group sum to zero.
    # Each branch's probabilities sum to one: the value gradients of a group
    # sum to the gate-weighted upstream gradient over the branches that have
    # keys (the compressed one only once a whole block is in the past).
    block, top_k, window = 16, 3, 20
    d = _data(90, 6, 2, 8, seed=7, batch=2)
    idx = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=block, top_k=top_k,
                          window=window)["idx"]
    g = nsa_bwd_ref.prefill_backward(d["q"], d["k"], d["v"], d["gates"], d["dout"], idx, block=block,
                                     top_k=top_k, window=window)
    np.testing.assert_allclose(g["dk"].sum(axis=1), 0.0, atol=1e-11)
    B, L, Hq, D = d["q"].shape
    has_cmp = (np.arange(L) + 1 >= block).astype(np.float64)  # [L]
    w = d["gates"][..., 1] + d["gates"][..., 2] + d["gates"][..., 0] * has_cmp[None, :, None]
    want = (w[..., None] * d["dout"]).reshape(B, L, 2, Hq // 2, D).sum(axis=(1, 3))
    np.testing.assert_allclose(g["dv"].sum(axis=1), want, atol=1e-11)


def test_rows_option_gives_the_whole_gradient_of_keys_only_those_rows_see():
    # The 64k GPU check compares dk / dv of the last block's keys with the
    # oracle run on the last 64 rows only: no earlier row sees those keys
    # (causal window, own-or-earlier blocks, complete block means), so the
    # restricted run must equal the full one there, and dq / dgates of the
    # given rows must equal the full run's.
    block, top_k, window = 16, 3, 20
    d = _data(80, 4, 2, 8, seed=9, top_k=top_k, window=window, block=block)
    idx = nsa_ref.prefill(d["q"], d["k"], d["v"], d["gates"], block=block, top_k=top_k, window=window)["idx"]
    full = nsa_bwd_ref.prefill_backward(d["q"], d["k"], d["v"], d["gates"], d["dout"], idx, block=block,
                                        top_k=top_k, window=window)
    last = np.arange(80 - block, 80)
    part = nsa_bwd_ref.prefill_backward(d["q"], d["k"], d["v"], d["gates"], d["dout"], idx, block=block,
                                        top_k=top_k, window=window, rows=last)
    for name in ("dk", "dv", "dq", "dgates"):
        np.testing.assert_allclose(part[name][:, last], full[name][:, last], rtol=0, atol=1e-12)
