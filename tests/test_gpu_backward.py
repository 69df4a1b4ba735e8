"""GPU parity of the prefill backward (nsa_bwd_prefill) against the float64 oracle.

Every gradient is compared element by element with the oracle on the same
seeded inputs and the same selection (the oracle's own forward selection, or a
seeded synthetic one: no oracle input comes from the GPU). The error measure
is max |gpu - oracle| / max |oracle| per tensor (relative to the tensor's own
largest gradient), bounded by 2e-2 for bf16 inputs (probabilities and score
gradients enter the matrix products rounded to bf16, relative step 2^-8, and
the sums run over thousands of terms) and 1e-4 for fp32 inputs. Where the
exact gradient vanishes (a softmax over a single key has zero derivative, so
dq and dk of a one-token sequence are 0), the GPU's value is a cancellation
residue of products of the size of dout . o; it is bounded by the same
tolerance times the largest |dout . o| (the gate gradient).

At the 64k bench shape the oracle checks sampled query rows (dq, dgates), the
keys of the last block (dk, dv: only the last 64 rows see them), and the
closed-form sum of the value gradients over all keys.
"""

import numpy as np
import pytest
import torch

from long_context_sparse_fwd_amd import inputs, nsa
from oracle import nsa_bwd_ref, nsa_ref
from tests.parity import dev as _up

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


def _err(got, want):
    """Largest deviation relative to the tensor's largest gradient."""
    return float(np.abs(got - want).max() / max(np.abs(want).max(), 1e-300))


VANISH = 1e-12  # an oracle gradient this small is zero up to float64 rounding


def _check_grads(tag, names, got, ref, dtype):
    scale = float(np.abs(ref["dgates"]).max())   # |dout . o|: the size of the products
    for nm, gv in zip(names, got):
        want = ref[nm]
        if np.abs(want).max() <= VANISH * max(scale, 1.0):
            e = float(np.abs(gv).max()) / max(scale, 1e-300)
            print(f"[bwd] {tag} {nm} vanishes: max |gpu| / max |dout . o| = {e:.2e}", flush=True)
        else:
            e = _err(gv, want)
            print(f"[bwd] {tag} {nm} relative err {e:.2e}", flush=True)
        assert e <= TOL[dtype], f"{tag} {nm} error {e}"


def _run(cfg, raw, dout_raw, idx, out_dtype=None):
    q, k, v, g = (_up(raw[n], cfg.dtype) for n in ("q", "k", "v", "gates"))
    dout = _up(dout_raw, out_dtype or cfg.dtype)
    grads = nsa.prefill_backward(q, k, v, g, dout, torch.from_numpy(idx).cuda(), top_k=cfg.top_k,
                                 window=cfg.window)
    torch.cuda.synchronize()
    return [x.cpu().numpy().astype(np.float64) for x in grads]


def _f64(raw, dtype):
    return {n: inputs.to_f64(raw[n], dtype) for n in ("q", "k", "v", "gates")}


CASES = [
    # name, B, L, Hq, G, D, dtype, top_k, window, selection source
    ("f32_tiny_heads", 1, 300, 4, 1, 64, "f32", 4, 128, "oracle"),
    ("bf16_ragged_batch", 2, 333, 8, 2, 128, "bf16", 4, 100, "oracle"),
    ("bf16_bench_heads", 1, 1100, 64, 4, 128, "bf16", 16, 512, "synthetic"),
    ("bf16_d64_short", 1, 130, 16, 4, 64, "bf16", 3, 40, "synthetic"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(case):
    name, B, L, Hq, G, D, dtype, n, w, src = case
    cfg = inputs.PrefillConfig(name, B, L, Hq, G, D, dtype, top_k=n, window=w, seed=11)
    print(f"[bwd] {cfg} selection={src}", flush=True)
    raw = inputs.make_prefill_inputs(cfg)
    dout_raw = inputs.make_dout(cfg)
    x = _f64(raw, dtype)
    dout = inputs.to_f64(dout_raw, dtype)
    if src == "oracle":
        idx = nsa_ref.prefill(x["q"], x["k"], x["v"], x["gates"], top_k=n, window=w)["idx"]
    else:
        idx = inputs.make_selection(cfg)
    ref = nsa_bwd_ref.prefill_backward(x["q"], x["k"], x["v"], x["gates"], dout, idx, top_k=n, window=w)
    got = _run(cfg, raw, dout_raw, idx)
    _check_grads(name, ("dq", "dk", "dv", "dgates"), got, ref, dtype)


EDGE = [
    # degenerate shapes: one token; one query head per KV head; top-k of one
    # (only the own block) and a window of one (only the token itself);
    # exactly one block (the compressed branch appears at the last token);
    # one token past it; window and top-k beyond the sequence
    ("one_token", 1, 1, 2, 2, 64, "f32", 2, 4),
    ("one_head_per_group", 1, 150, 3, 3, 64, "bf16", 2, 30),
    ("topk1_window1", 1, 200, 4, 1, 128, "bf16", 1, 1),
    ("exactly_one_block", 1, 64, 4, 2, 128, "f32", 2, 16),
    ("one_block_plus_one", 2, 65, 8, 2, 64, "bf16", 3, 8),
    ("window_and_topk_past_length", 1, 190, 4, 2, 64, "f32", 8, 4096),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_backward_edge_cases(case):
    name, B, L, Hq, G, D, dtype, n, w = case
    cfg = inputs.PrefillConfig(name, B, L, Hq, G, D, dtype, top_k=n, window=w, seed=13)
    print(f"[bwd] {cfg}", flush=True)
    raw = inputs.make_prefill_inputs(cfg)
    dout_raw = inputs.make_dout(cfg)
    x = _f64(raw, dtype)
    dout = inputs.to_f64(dout_raw, dtype)
    idx = nsa_ref.prefill(x["q"], x["k"], x["v"], x["gates"], top_k=n, window=w)["idx"]
    ref = nsa_bwd_ref.prefill_backward(x["q"], x["k"], x["v"], x["gates"], dout, idx, top_k=n, window=w)
    got = _run(cfg, raw, dout_raw, idx)
    _check_grads(name, ("dq", "dk", "dv", "dgates"), got, ref, dtype)


@pytest.mark.parametrize("case", [CASES[0], CASES[1]], ids=["f32", "bf16"])
def test_forward_save_and_saved_backward(case):
    # nsa_fwd_prefill_save: out and idx bit for bit those of nsa_fwd_prefill,
    # the kept selected-branch output and log-sum-exp equal to the oracle's;
    # nsa_bwd_prefill_saved from them (the oracle's selection injected)
    # matches the backward oracle like the plain backward does.
    name, B, L, Hq, G, D, dtype, n, w, _ = case
    cfg = inputs.PrefillConfig(name, B, L, Hq, G, D, dtype, top_k=n, window=w, seed=14)
    print(f"[bwd saved] {cfg}", flush=True)
    raw = inputs.make_prefill_inputs(cfg)
    q, k, v, g = (_up(raw[nm], dtype) for nm in ("q", "k", "v", "gates"))
    out0, idx0 = nsa.prefill(q, k, v, g, top_k=n, window=w, return_idx=True)
    out1, idx1, _ = nsa.prefill_save(q, k, v, g, top_k=n, window=w)
    torch.cuda.synchronize()
    assert torch.equal(idx0, idx1)
    assert torch.equal(out0.view(torch.int16) if dtype == "bf16" else out0,
                       out1.view(torch.int16) if dtype == "bf16" else out1)
    x = _f64(raw, dtype)
    orc = nsa_ref.prefill(x["q"], x["k"], x["v"], x["gates"], top_k=n, window=w, branches=True)
    _, _, (o_slc, lse_slc) = nsa.prefill_save(q, k, v, g, top_k=n, window=w,
                                              idx=torch.from_numpy(orc["idx"]).cuda(), inject=True)
    torch.cuda.synchronize()
    e_o = float(np.abs(o_slc.float().cpu().numpy() - orc["o_slc"]).max())
    lg, lr = lse_slc.cpu().numpy().astype(np.float64), orc["lse_slc"]
    assert np.array_equal(np.isinf(lg), np.isinf(lr))
    fin = np.isfinite(lr)
    e_l = float(np.abs(lg[fin] - lr[fin]).max())
    print(f"[bwd saved] {name} o_slc err {e_o:.2e} lse_slc err {e_l:.2e}", flush=True)
    assert e_o <= (2e-2 if dtype == "bf16" else 1e-4) and e_l <= 1e-4
    dout_raw = inputs.make_dout(cfg)
    ref = nsa_bwd_ref.prefill_backward(x["q"], x["k"], x["v"], x["gates"], inputs.to_f64(dout_raw, dtype),
                                       orc["idx"], top_k=n, window=w)
    grads = nsa.prefill_backward(q, k, v, g, _up(dout_raw, dtype), torch.from_numpy(orc["idx"]).cuda(), top_k=n,
                                 window=w, saved=(o_slc, lse_slc))
    torch.cuda.synchronize()
    _check_grads(f"saved {name}", ("dq", "dk", "dv", "dgates"),
                 [gt.cpu().numpy().astype(np.float64) for gt in grads], ref, dtype)


def test_backward_with_fp32_upstream_gradient_and_odd_selection():
    # bf16 inputs with an fp32 output (so an fp32 dout), and an injected
    # selection with repeats, entries past the own block and negative entries
    # (a set of blocks, as in the forward).
    cfg = inputs.PrefillConfig("odd", 1, 200, 16, 4, 64, "bf16", top_k=4, window=50, seed=12)
    print(f"[bwd] {cfg}", flush=True)
    raw = inputs.make_prefill_inputs(cfg)
    dout_raw = inputs.make_dout(cfg, "f32")
    idx = inputs.make_selection(cfg)
    idx[0, 70:90, 1, 3] = idx[0, 70:90, 1, 0]
    idx[0, 100:110, 2, 2] = 3
    idx[0, 120:130, 0, :] = -7
    x = _f64(raw, "bf16")
    ref = nsa_bwd_ref.prefill_backward(x["q"], x["k"], x["v"], x["gates"], inputs.to_f64(dout_raw, "f32"), idx,
                                       top_k=4, window=50)
    got = _run(cfg, raw, dout_raw, idx, out_dtype="f32")
    _check_grads('odd', ("dq", "dk", "dv", "dgates"), got, ref, "bf16")


def test_backward_at_64k_sampled_rows_last_block_and_value_sum():
    cfg = inputs.CONFIGS["p64k"]
    print(f"[bwd] {cfg}", flush=True)
    raw = inputs.make_prefill_inputs(cfg)
    dout_raw = inputs.make_dout(cfg)
    idx = inputs.make_selection(cfg)
    dq, dk, dv, dgates = _run(cfg, raw, dout_raw, idx)
    x = _f64(raw, "bf16")
    dout = inputs.to_f64(dout_raw, "bf16")
    L = cfg.seqlen
    rng = np.random.default_rng(3)
    rows = np.sort(np.concatenate([rng.choice(L - 64, 10, replace=False), [0, 63, 64, 4095]]))
    ref = nsa_bwd_ref.prefill_backward(x["q"], x["k"], x["v"], x["gates"], dout, idx, top_k=cfg.top_k,
                                       window=cfg.window, rows=rows)
    for nm, gv in (("dq", dq), ("dgates", dgates)):
        e = _err(gv[:, rows], ref[nm][:, rows])
        print(f"[bwd] p64k sampled {nm} err {e:.2e}", flush=True)
        assert e <= TOL["bf16"], f"{nm} error {e}"
    last = np.arange(L - 64, L)
    ref = nsa_bwd_ref.prefill_backward(x["q"], x["k"], x["v"], x["gates"], dout, idx, top_k=cfg.top_k,
                                       window=cfg.window, rows=last)
    for nm, gv in (("dk", dk), ("dv", dv), ("dq", dq)):
        e = _err(gv[:, last], ref[nm][:, last])
        print(f"[bwd] p64k last block {nm} err {e:.2e}", flush=True)
        assert e <= TOL["bf16"], f"{nm} error {e}"
    # sum of the value gradients of a group over all keys: the gate-weighted
    # upstream gradient of the branches that have keys
    B, _, Hq, D = x["q"].shape
    G = cfg.n_kv_heads
    has_cmp = (np.arange(L) + 1 >= 64).astype(np.float64)
    wgt = x["gates"][..., 1] + x["gates"][..., 2] + x["gates"][..., 0] * has_cmp[None, :, None]
    want = (wgt[..., None] * dout).reshape(B, L, G, Hq // G, D).sum(axis=(1, 3))
    e = _err(dv.sum(axis=1), want)
    print(f"[bwd] p64k value-gradient sum err {e:.2e}", flush=True)
    assert e <= TOL["bf16"]
