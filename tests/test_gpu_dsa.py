"""GPU parity of nsa_dsa_prefill (token-level sparse attention with a ReLU
indexer) against the float64 oracle (oracle/dsa_ref.py), through the C ABI.

Protocol, as for the block-sparse forward:
* Check A (tokens): every row's chosen set equals the oracle's, unless the
  oracle's top_k-th and (top_k+1)-th scores differ by less than 1e-4; such a
  row must still hold every token scoring more than 1e-4 above the oracle's
  top_k-th score and only tokens scoring at least its (top_k+1)-th minus 1e-4.
  Rows are ascending with -1 padding and hold min(top_k, t + 1) tokens.
* Check B: rows whose set matches against the oracle output; differing
  (excused) rows against the oracle run with the GPU's selection injected.
* Check C: the GPU with the oracle's selection injected against the oracle.
* Tolerance: max-abs 1e-4 for fp32 inputs, 2e-2 for bf16 (fp32 and bf16 output).
"""

import numpy as np
import pytest
import torch

from long_context_sparse_fwd_amd import inputs, nsa
from oracle import dsa_ref
from tests.parity import EXCUSE, TOL, Lazy, dev, maxabs

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "qi", "ki", "w")


def check_tokens(gi, oi, gap, scores, rows, k):
    """Check A over [N, k] rows; returns (exact, excused_differing, failures)."""
    exact, excused, bad = 0, 0, []
    for r in range(gi.shape[0]):
        t = int(rows[r])
        g = [int(x) for x in gi[r]]
        o = [int(x) for x in oi[r]]
        valid = [x for x in g if x >= 0]
        if (g != valid + [-1] * (k - len(valid)) or valid != sorted(set(valid)) or len(valid) != min(k, t + 1)
                or any(x > t for x in valid)):
            bad.append((r, "malformed row", g[:8]))
            continue
        if g == o:
            exact += 1
            continue
        if not gap[r] < EXCUSE:
            bad.append((r, f"set differs with gap {gap[r]:.3g}"))
            continue
        sc = scores[r, : t + 1]
        ranked = np.sort(sc)[::-1]
        s_hi, s_lo = ranked[k - 1], ranked[k]
        gs = set(valid)
        ok = all(s in gs for s in range(t + 1) if sc[s] > s_hi + EXCUSE)
        ok &= all(sc[s] >= s_lo - EXCUSE for s in gs)
        if ok:
            excused += 1
        else:
            bad.append((r, "excused row outside the tie band"))
    return exact, excused, bad


def _rows_of(t, rows):
    return t[:, torch.as_tensor(rows, device=t.device)].float().cpu().numpy().astype(np.float64)


def run_dsa(cfg, rows=None, check_c=True, w_override=None):
    raw = inputs.make_dsa_inputs(cfg)
    if w_override is not None:
        raw["w"] = w_override(raw["w"])
    ts = [dev(raw[n], cfg.dtype) for n in NAMES]
    print(f"[dsa] {cfg}", flush=True)
    out, idx = nsa.dsa_prefill(*ts, top_k=cfg.top_k, out_dtype=torch.float32, return_idx=True)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    B, L, k = gi.shape
    rows = np.arange(L) if rows is None else np.asarray(sorted(set(int(r) for r in rows if 0 <= r < L)))
    lz = {n: Lazy(raw[n], cfg.dtype) for n in NAMES}
    orc = dsa_ref.prefill(*(lz[n] for n in NAMES), top_k=k, rows=rows, scores=True)
    gsel = gi[:, rows]
    rr = np.broadcast_to(rows[None, :], gsel.shape[:2]).reshape(-1)
    exact, excused, bad = check_tokens(gsel.reshape(-1, k), orc["idx"].reshape(-1, k), orc["gap"].reshape(-1),
                                       orc["scores"].reshape(-1, L), rr, k)
    assert not bad, f"selection mismatches: {bad[:5]}"
    expect = orc["out"].copy()
    for b, r in np.argwhere(np.any(gsel != orc["idx"], axis=2)):
        inj = np.zeros((1, L, k), np.int32)
        inj[0, rows[r]] = gi[b, rows[r]]
        sub = {n: Lazy(raw[n][b:b + 1], cfg.dtype) for n in NAMES}
        expect[b, r] = dsa_ref.prefill(*(sub[n] for n in NAMES), top_k=k, rows=[rows[r]], inject_idx=inj)["out"][0, 0]
    err_b = maxabs(_rows_of(out, rows), expect)
    assert err_b <= TOL[cfg.dtype], f"free-running output error {err_b}"
    err_c = None
    if check_c:
        inj = gi.copy()
        inj[:, rows] = orc["idx"]
        oc = nsa.dsa_prefill(*ts, top_k=k, out_dtype=torch.float32, idx=torch.from_numpy(inj).cuda(), inject=True)[0]
        torch.cuda.synchronize()
        err_c = maxabs(_rows_of(oc, rows), orc["out"])
        assert err_c <= TOL[cfg.dtype], f"injected-selection output error {err_c}"
    err_16 = None
    if cfg.dtype == "bf16":
        o16, i16 = nsa.dsa_prefill(*ts, top_k=k, out_dtype=torch.bfloat16, return_idx=True)
        torch.cuda.synchronize()
        assert torch.equal(i16, idx)
        assert torch.equal(o16.view(torch.int16), out.to(torch.bfloat16).view(torch.int16))
        err_16 = maxabs(_rows_of(o16, rows), expect)
        assert err_16 <= TOL["bf16"], f"bf16-output error {err_16}"
    print(f"  rows={len(rows)} exact={exact} excused={excused} errB={err_b:.3g} errC={err_c} bf16 errB={err_16}",
          flush=True)
    return gi, out


CASES = [
    # name, B, L, Hq, G, D, Hi, Di, dtype, top_k
    ("f32-small", 1, 300, 4, 1, 64, 4, 64, "f32", 32),
    ("f32-d128-gqa", 1, 260, 8, 2, 128, 8, 128, "f32", 40),
    ("bf16-mqa-64heads", 1, 1500, 64, 1, 128, 16, 128, "bf16", 256),
    ("bf16-gqa-4x16", 1, 900, 64, 4, 128, 16, 128, "bf16", 128),
    ("bf16-gqa-2x32", 2, 700, 64, 2, 128, 16, 64, "bf16", 100),
    ("bf16-hg3-d64", 1, 500, 6, 2, 64, 5, 64, "bf16", 50),
    ("bf16-topk-past-length", 1, 200, 16, 1, 64, 8, 64, "bf16", 256),
    ("bf16-topk1", 1, 150, 16, 1, 128, 16, 128, "bf16", 1),
    ("bf16-one-token", 1, 1, 16, 1, 128, 16, 128, "bf16", 8),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_dsa_matches_oracle(case):
    name, B, L, Hq, G, D, Hi, Di, dtype, k = case
    run_dsa(inputs.DsaConfig(name, B, L, Hq, G, D, Hi, Di, dtype, top_k=k, seed=31))


def test_dsa_all_ties_pick_the_lowest_tokens():
    # zero indexer head weights: every score is 0, every row takes its first
    # top_k tokens
    cfg = inputs.DsaConfig("ties", 1, 400, 16, 1, 64, 4, 64, "bf16", top_k=64, seed=32)
    gi, _ = run_dsa(cfg, w_override=lambda w: np.zeros_like(w))
    for t in (0, 63, 64, 399):
        n = min(64, t + 1)
        assert list(gi[0, t, :n]) == list(range(n))


def test_dsa_injected_selection_is_a_set_of_tokens():
    cfg = inputs.DsaConfig("inject", 2, 300, 16, 1, 64, 4, 64, "bf16", top_k=24, seed=33)
    raw = inputs.make_dsa_inputs(cfg)
    ts = [dev(raw[n], cfg.dtype) for n in NAMES]
    rng = np.random.default_rng(3)
    inj = rng.integers(-3, cfg.seqlen + 3, size=(cfg.batch, cfg.seqlen, cfg.top_k)).astype(np.int32)
    inj[..., 1] = inj[..., 0]
    inj[:, ::7] = -1
    out = nsa.dsa_prefill(*ts, top_k=cfg.top_k, out_dtype=torch.float32, idx=torch.from_numpy(inj).cuda(),
                          inject=True)[0]
    torch.cuda.synchronize()
    lz = {n: Lazy(raw[n], cfg.dtype) for n in NAMES}
    orc = dsa_ref.prefill(*(lz[n] for n in NAMES), top_k=cfg.top_k, inject_idx=inj)
    err = maxabs(out.cpu().numpy().astype(np.float64), orc["out"])
    print(f"[dsa inject] err {err:.3g}", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("name,n_rows", [("dsa8k", 160), ("dsa64k", 48)])
def test_dsa_full_size_sampled_rows(name, n_rows):
    cfg = inputs.DSA_CONFIGS[name]
    L = cfg.seqlen
    rng = np.random.default_rng(7)
    rows = sorted({0, 1, 2046, 2047, 2048, 2049, L // 2, L - 2, L - 1, *rng.integers(0, L, n_rows).tolist()})
    run_dsa(cfg, rows=rows)


def test_dsa_rows_past_the_candidate_capacity_with_ties():
    # zero indexer head weights: every score is 0. Rows of up to 3584 tokens
    # keep all their keys as candidates; longer rows pass every key through
    # the sampled threshold, overflow the 3584-key candidate list and are
    # redone by the exact pass. Both must take the first top_k tokens.
    cfg = inputs.DsaConfig("redo-ties", 1, 4700, 16, 1, 64, 4, 64, "bf16", top_k=64, seed=34)
    rows = [0, 63, 64, 4094, 4095, 4096, 4097, 4400, 4699]
    gi, _ = run_dsa(cfg, rows=rows, w_override=lambda w: np.zeros_like(w))
    for t in rows:
        n = min(64, t + 1)
        assert list(gi[0, t, :n]) == list(range(n)) and all(x == -1 for x in gi[0, t, n:])


def test_dsa_sampled_threshold_rows():
    # rows longer than the 3584-key candidate list take the sampled threshold;
    # every row from 4000 on is checked against the oracle, with top_k of
    # 256 and of the largest supported 2048
    for k in (256, 2048):
        cfg = inputs.DsaConfig(f"sampled-k{k}", 1, 5200, 16, 1, 64, 8, 64, "bf16", top_k=k, seed=35)
        run_dsa(cfg, rows=list(range(4000, 5200)), check_c=False)
