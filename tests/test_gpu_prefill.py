"""GPU parity of nsa_fwd_prefill against the float64 oracle (through the C ABI).

Small cases are compared on every row; the 8k / 32k / 64k workloads run in
full on the GPU, exactly as the benchmark launches them, and are compared on
sampled rows that the oracle computes one by one, plus row-format properties
that must hold on every row.
"""

import numpy as np
import pytest
import torch

from long_context_sparse_fwd_amd import inputs, nsa
from oracle import nsa_ref
from tests.parity import TOL, Lazy, check_indices, dev, maxabs

pytestmark = pytest.mark.gpu


def _upload(cfg, raw):
    return [dev(raw[n], cfg.dtype) for n in ("q", "k", "v", "gates")]


def _oracle(cfg, raw, rows, inject=None):
    lz = {n: Lazy(raw[n], cfg.dtype) for n in raw}
    return nsa_ref.prefill(lz["q"], lz["k"], lz["v"], lz["gates"], block=cfg.block, top_k=cfg.top_k,
                           window=cfg.window, rows=rows, inject_idx=inject, scores=inject is None)


def check_rows(cfg, raw, rows, go, gi):
    """Checks A and B for the query positions ``rows`` of every sequence of
    ``raw`` (host arrays [B, L, ...]): ``go`` [B, R, Hq, D] and ``gi``
    [B, R, G, n] are the GPU's output and selection at those rows. Returns
    (oracle result, expected output per row, counts, Check B error)."""
    n = cfg.top_k
    orc = _oracle(cfg, raw, rows)
    own = np.broadcast_to((np.asarray(rows) // cfg.block)[None, :, None], gi.shape[:3])
    sc = orc["scores"]
    sc = sc.reshape(-1, sc.shape[-1]) if sc.shape[-1] else np.zeros((gi.size // n, 1))
    exact, excused, bad = check_indices(gi.reshape(-1, n), orc["idx"].reshape(-1, n), orc["gap"].reshape(-1), sc,
                                        own.reshape(-1), n)
    assert not bad, f"index mismatches: {bad[:5]}"
    # Check B: matching rows against the oracle, differing (excused) rows
    # against the oracle re-run with the GPU's selection injected
    expect = orc["out"].copy()
    for b, r in np.argwhere(np.any(gi != orc["idx"], axis=(2, 3))):
        inj = np.zeros((1, raw["k"].shape[1], cfg.n_kv_heads, n), np.int32)
        inj[0, rows[r]] = gi[b, r]
        re = _oracle(cfg, {kk: vv[b:b + 1] for kk, vv in raw.items()}, [rows[r]], inject=inj)
        expect[b, r] = re["out"][0, 0]
    err_b = maxabs(go, expect)
    return orc, expect, (exact, excused), err_b


def _rows_of(t: torch.Tensor, rows) -> np.ndarray:
    return t[:, torch.as_tensor(rows, device=t.device)].float().cpu().numpy().astype(np.float64)


def run_case(cfg, rows=None, check_c=True):
    """Checks A, B and C for one prefill workload; for bf16 inputs also the
    bf16-output instance (the one the benchmark times), which must be the
    fp32 output rounded once and meet the same bound. Returns a small report."""
    raw = inputs.make_prefill_inputs(cfg)
    q, k, v, g = _upload(cfg, raw)
    print(f"[prefill] {cfg}", flush=True)
    out, idx = nsa.prefill(q, k, v, g, top_k=cfg.top_k, window=cfg.window, out_dtype=torch.float32,
                           return_idx=True)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    B, L, G, n = gi.shape
    rows = np.arange(L) if rows is None else np.asarray(sorted(set(int(r) for r in rows if 0 <= r < L)))
    go = _rows_of(out, rows)
    orc, expect, (exact, excused), err_b = check_rows(cfg, raw, rows, go, gi[:, rows])
    assert err_b <= TOL[cfg.dtype], f"free-running output error {err_b}"

    err_c = inj_t = None
    if check_c:
        inj = gi.copy()
        inj[:, rows] = orc["idx"]
        inj_t = torch.from_numpy(inj).cuda()
        out_c = nsa.prefill(q, k, v, g, top_k=cfg.top_k, window=cfg.window, out_dtype=torch.float32, idx=inj_t,
                            inject=True)[0]
        torch.cuda.synchronize()
        err_c = maxabs(_rows_of(out_c, rows), orc["out"])
        del out_c
        assert err_c <= TOL[cfg.dtype], f"injected-index output error {err_c}"

    err_b16 = err_c16 = None
    if cfg.dtype == "bf16":
        o16, i16 = nsa.prefill(q, k, v, g, top_k=cfg.top_k, window=cfg.window, out_dtype=torch.bfloat16,
                               return_idx=True)
        torch.cuda.synchronize()
        assert torch.equal(i16, idx), "the selection depends on the output type"
        # one rounding (to nearest even) of the same fp32 sum of the three branches
        assert torch.equal(o16.view(torch.int16), out.to(torch.bfloat16).view(torch.int16)), \
            "bf16 output is not the fp32 output rounded once"
        err_b16 = maxabs(_rows_of(o16, rows), expect)
        assert err_b16 <= TOL["bf16"], f"bf16-output free-running error {err_b16}"
        del o16
        if check_c:
            oc16 = nsa.prefill(q, k, v, g, top_k=cfg.top_k, window=cfg.window, out_dtype=torch.bfloat16, idx=inj_t,
                               inject=True)[0]
            torch.cuda.synchronize()
            err_c16 = maxabs(_rows_of(oc16, rows), orc["out"])
            del oc16
            assert err_c16 <= TOL["bf16"], f"bf16-output injected-index error {err_c16}"
    fmt = lambda e: "-" if e is None else f"{e:.3g}"
    print(f"  rows={len(rows)} exact={exact} excused={excused} fp32-out errB={fmt(err_b)} errC={fmt(err_c)}"
          f" bf16-out errB={fmt(err_b16)} errC={fmt(err_c16)}", flush=True)
    return {"gpu_idx": gi, "gpu_out": go, "rows": rows, "oracle": orc, "tensors": (q, k, v, g),
            "errors": {"fp32_out_B": err_b, "fp32_out_C": err_c, "bf16_out_B": err_b16, "bf16_out_C": err_c16}}


def assert_rows_well_formed(gi, block):
    """Every row: ascending valid indices, -1 padding, own block present, range [0, own]."""
    B, L, G, n = gi.shape
    own = (np.arange(L) // block)[None, :, None]
    valid = gi >= 0
    cnt = valid.sum(-1)
    assert np.all(cnt == np.minimum(n, own + 1))
    assert np.all(valid[..., :-1] | ~valid[..., 1:])            # padding only at the end
    both = valid[..., 1:] & valid[..., :-1]
    assert np.all(np.where(both, np.diff(gi, axis=-1) > 0, True))   # strictly ascending
    assert np.all(gi <= own[..., None])
    assert np.all(np.any(gi == own[..., None], axis=-1))


# ------------------------------------------------------------------ full-row cases

def test_tiny_fp32_config():
    run_case(inputs.CONFIGS["tiny"])


@pytest.mark.parametrize("cfg", [
    inputs.PrefillConfig("bf16-ragged", 1, 1381, 32, 2, 128, "bf16", top_k=16, window=512),
    inputs.PrefillConfig("bf16-d64-b2", 2, 777, 16, 2, 64, "bf16", top_k=5, window=100),
    inputs.PrefillConfig("bf16-hg3", 1, 300, 6, 2, 128, "bf16", top_k=3, window=70),
    inputs.PrefillConfig("f32-hg1", 1, 333, 2, 2, 64, "f32", top_k=4, window=33),
    inputs.PrefillConfig("f32-d128", 1, 260, 8, 1, 128, "f32", top_k=2, window=64),
], ids=lambda c: c.name)
def test_prefill_full_rows(cfg):
    run_case(cfg)


@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 127, 128, 129])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_short_sequences(L, dtype):
    run_case(inputs.PrefillConfig(f"short{L}", 1, L, 16, 1, 64, dtype, top_k=3, window=40))


@pytest.mark.parametrize("top_k,window", [(1, 1), (64, 1), (2, 10000), (40, 3)])
def test_prefill_parameter_extremes(top_k, window):
    run_case(inputs.PrefillConfig(f"ext{top_k}-{window}", 1, 700, 16, 2, 64, "bf16", top_k=top_k,
                                  window=window))


# ------------------------------------------------------------------ full-size workloads

def _sample_rows(L, per_block=1, seed=0, n_random=0):
    """Query rows for a full-size check: ``per_block`` rows at random offsets
    inside every 64-token block (so every position mod 64 and every tile of
    the kernels is reached over the blocks), fixed rows at block and tile
    edges (the compressed kernel takes 16 tokens per workgroup, the selected
    one 8), the ends, and the neighbourhoods of the points where the
    selected-branch kernel divides one long sequence between two XCDs (half
    of its tiles, or 57 % of them past 32k tokens), plus ``n_random`` rows
    drawn uniformly."""
    rng = np.random.default_rng(seed)
    nb = -(-L // 64)
    rows = [64 * j + int(x) for j in range(nb) for x in rng.integers(0, 64, per_block)]
    fixed = [0, 1, 7, 8, 15, 16, 62, 63, 64, 65, 127, 511, 512, 513, 4095, 4096, L - 65, L - 64, L - 2, L - 1]
    for split in (L // 2, (L // 8 * 57 + 99) // 100 * 8):
        fixed += [split - 9, split - 8, split - 1, split, split + 7, split + 8]
    rnd = rng.integers(0, L, n_random).tolist()
    return sorted(set(r for r in rows + fixed + rnd if 0 <= r < L))


@pytest.mark.parametrize("name,per_block", [("p8k", 2), ("p32k", 1), ("p64k", 1)])
def test_full_size_prefill_sampled_rows(name, per_block):
    cfg = inputs.CONFIGS[name]
    rep = run_case(cfg, rows=_sample_rows(cfg.seqlen, per_block=per_block), check_c=True)
    assert_rows_well_formed(rep["gpu_idx"], cfg.block)
    assert np.all(np.isfinite(rep["gpu_out"]))


@pytest.mark.parametrize("L", [70000, 110000, 200000])
def test_long_prefill_other_compressed_layouts(L):
    """Past 64k tokens (D 128, bf16) the block scores leave less LDS for the
    compressed kernel's stage: 70000 runs it with 8 waves and the low parts
    of the K means read from L2, 110000 with 4 waves per workgroup, 200000
    with 2. Sixteen query heads in one group keep the host side small;
    compared on sampled rows."""
    cfg = inputs.PrefillConfig(f"long{L}", 1, L, 16, 1, 128, "bf16", top_k=16, window=512)
    rep = run_case(cfg, rows=_sample_rows(L, per_block=0, n_random=64), check_c=True)
    assert_rows_well_formed(rep["gpu_idx"], cfg.block)
    assert np.all(np.isfinite(rep["gpu_out"]))


def test_chunked_prefill_matches_oracle_and_whole_prefill_rows():
    """nsa_fwd_prefill_chunk over consecutive chunks at unaligned offsets, each
    seeing the context only up to its end: rows of every chunk are checked
    against the oracle directly (Checks A and B, fp32 and bf16 output), and
    every row equals the whole prefill's row bit for bit (output and
    selection, computed and injected)."""
    cfg = inputs.PrefillConfig("chunks", 2, 3001, 32, 2, 128, "bf16", top_k=8, window=300)
    raw = inputs.make_prefill_inputs(cfg)
    q, k, v, g = _upload(cfg, raw)
    print(f"[prefill chunks] {cfg}", flush=True)
    fo, fi = nsa.prefill(q, k, v, g, top_k=8, window=300, out_dtype=torch.float32, return_idx=True)
    bounds = [0, 1, 700, 1029, 2048, 2999, 3001]
    rng = np.random.default_rng(5)
    for t0, t1 in zip(bounds[:-1], bounds[1:]):
        args = (q[:, t0:t1], k[:, :t1], v[:, :t1], g[:, t0:t1], t0)
        o, i = nsa.prefill_chunk(*args, top_k=8, window=300, out_dtype=torch.float32, return_idx=True)
        o16 = nsa.prefill_chunk(*args, top_k=8, window=300, out_dtype=torch.bfloat16)
        oi = nsa.prefill_chunk(*args, top_k=8, window=300, out_dtype=torch.float32,
                               idx=fi[:, t0:t1].contiguous(), inject=True)[0]
        torch.cuda.synchronize()
        assert torch.equal(i, fi[:, t0:t1]), (t0, t1)
        assert torch.equal(o, fo[:, t0:t1]), (t0, t1)
        assert torch.equal(oi, fo[:, t0:t1]), (t0, t1)
        # the chunk's own rows against the oracle over the context [0, t1)
        rows = sorted({t0, t1 - 1, *rng.integers(t0, t1, 24).tolist()})
        ctx = {n: raw[n][:, :t1] for n in raw}
        loc = [r - t0 for r in rows]
        gi = i.cpu().numpy()[:, loc]
        _, expect, (ex, exc), err = check_rows(cfg, ctx, rows, _rows_of(o, loc), gi)
        err16 = maxabs(_rows_of(o16, loc), expect)
        print(f"  chunk [{t0}, {t1}) rows={len(rows)} exact={ex} excused={exc} errB={err:.3g} bf16 errB={err16:.3g}",
              flush=True)
        assert err <= TOL["bf16"] and err16 <= TOL["bf16"], (t0, t1, err, err16)


def test_varlen_prefill_matches_oracle_per_sequence():
    """nsa_fwd_prefill_varlen with mixed context lengths and query offsets in
    one call (including a query range cut by the row count and an invalid
    length): each sequence's rows are checked against the oracle run on that
    sequence alone at its own length (Checks A and B, fp32 and bf16 output),
    equal the chunked prefill of that sequence bit for bit, and every other
    row is left untouched."""
    cfg = inputs.PrefillConfig("varlen", 4, 2100, 16, 2, 128, "bf16", top_k=8, window=300)
    raw = inputs.make_prefill_inputs(cfg)
    q, k, v, g = _upload(cfg, raw)
    print(f"[prefill varlen] {cfg}", flush=True)
    B, L, Hq, D = q.shape
    lens, offs, R = [2100, 1500, 777, 3000], [0, 1000, 700, 0], 1400
    qv = torch.zeros((B, R, Hq, D), dtype=q.dtype, device=q.device)
    gv = torch.zeros((B, R, Hq, 3), dtype=g.dtype, device=g.device)
    rows = [min(ln, o + R) - o if ln <= L else 0 for ln, o in zip(lens, offs)]
    for b in range(B):
        if rows[b]:
            qv[b, :rows[b]] = q[b, offs[b]:offs[b] + rows[b]]
            gv[b, :rows[b]] = g[b, offs[b]:offs[b] + rows[b]]
    sl = torch.tensor(lens, dtype=torch.int32, device=q.device)
    so = torch.tensor(offs, dtype=torch.int32, device=q.device)
    out, idx = nsa.prefill_varlen(qv, k, v, gv, sl, so, top_k=8, window=300, out_dtype=torch.float32,
                                  return_idx=True)
    o16 = nsa.prefill_varlen(qv, k, v, gv, sl, so, top_k=8, window=300, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert rows == [1400, 500, 77, 0]
    rng = np.random.default_rng(6)
    for b in range(B):
        n, t0 = rows[b], offs[b]
        if n:
            ro, ri = nsa.prefill_chunk(q[b:b + 1, t0:t0 + n], k[b:b + 1, :t0 + n], v[b:b + 1, :t0 + n],
                                       g[b:b + 1, t0:t0 + n], t0, top_k=8, window=300, out_dtype=torch.float32,
                                       return_idx=True)
            torch.cuda.synchronize()
            assert torch.equal(out[b, :n], ro[0]), b
            assert torch.equal(idx[b, :n], ri[0]), b
            # sequence b alone, context [0, lens[b]), against the oracle
            pos = sorted({t0, t0 + n - 1, *rng.integers(t0, t0 + n, 20).tolist()})
            loc = [p - t0 for p in pos]
            seq = {nm: raw[nm][b:b + 1, :lens[b]] for nm in raw}
            gi = idx[b:b + 1].cpu().numpy()[:, loc]
            _, expect, (ex, exc), err = check_rows(cfg, seq, pos, _rows_of(out[b:b + 1], loc), gi)
            err16 = maxabs(_rows_of(o16[b:b + 1], loc), expect)
            print(f"  sequence {b} (length {lens[b]}, queries from {t0}) rows={len(pos)} exact={ex} excused={exc} "
                  f"errB={err:.3g} bf16 errB={err16:.3g}", flush=True)
            assert err <= TOL["bf16"] and err16 <= TOL["bf16"], (b, err, err16)
        assert torch.all(out[b, n:] == 0) and torch.all(idx[b, n:] == -1), b


# ------------------------------------------------------------------ properties

def test_prefill_is_deterministic():
    cfg = inputs.PrefillConfig("det", 1, 2000, 64, 4, 128, "bf16", top_k=16, window=512)
    raw = inputs.make_prefill_inputs(cfg)
    q, k, v, g = _upload(cfg, raw)
    ref = nsa.prefill(q, k, v, g, top_k=16, window=512, return_idx=True)
    for _ in range(10):
        o, i = nsa.prefill(q, k, v, g, top_k=16, window=512, return_idx=True)
        assert torch.equal(o.view(torch.int16), ref[0].view(torch.int16))
        assert torch.equal(i, ref[1])


def test_prefill_writes_only_its_outputs():
    # out and idx are views inside larger buffers filled with a sentinel: the
    # call must leave everything around them untouched
    cfg = inputs.PrefillConfig("guard", 1, 333, 16, 2, 64, "bf16", top_k=4, window=50)
    raw = inputs.make_prefill_inputs(cfg)
    q, k, v, g = _upload(cfg, raw)
    big = torch.full((3, 333, 16, 64), 7.25, dtype=torch.float32, device="cuda")
    ibig = torch.full((3 * 333 * 2 * 4,), -77, dtype=torch.int32, device="cuda")
    out = big[1:2]
    idx = ibig[333 * 2 * 4: 2 * 333 * 2 * 4].view(1, 333, 2, 4)
    nsa.prefill(q, k, v, g, top_k=4, window=50, out=out, idx=idx)
    torch.cuda.synchronize()
    assert torch.all(big[0] == 7.25) and torch.all(big[2] == 7.25)
    assert torch.all(ibig[: 333 * 8] == -77) and torch.all(ibig[2 * 333 * 8:] == -77)
    assert torch.all(torch.isfinite(out))


def test_strided_inputs():
    # q/k/v/gates/out as views of packed buffers (non-default strides)
    cfg = inputs.PrefillConfig("strided", 1, 400, 16, 2, 64, "bf16", top_k=4, window=60)
    raw = inputs.make_prefill_inputs(cfg)
    q, k, v, g = _upload(cfg, raw)
    ref, ridx = nsa.prefill(q, k, v, g, top_k=4, window=60, out_dtype=torch.float32, return_idx=True)
    qkv = torch.zeros((1, 400, 16 + 2 + 2, 64), dtype=torch.bfloat16, device="cuda")
    qkv[:, :, :16] = q
    qkv[:, :, 16:18] = k
    qkv[:, :, 18:20] = v
    gb = torch.zeros((1, 400, 16, 5), dtype=torch.bfloat16, device="cuda")
    gb[..., 1:4] = g
    ob = torch.zeros((1, 400, 16, 72), dtype=torch.float32, device="cuda")
    out, idx = nsa.prefill(qkv[:, :, :16], qkv[:, :, 16:18], qkv[:, :, 18:20], gb[..., 1:4], top_k=4,
                           window=60, out=ob[..., :64], return_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(idx, ridx)
    assert torch.equal(out, ref)
    assert torch.all(ob[..., 64:] == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_injected_selection_with_repeats_and_unusable_entries(dtype):
    # an injected selection is a set of blocks: repeats, negative entries and
    # entries after the own block add nothing; rows with no usable entry get a
    # selected branch of 0. Every row is compared with the oracle given the
    # same injection.
    cfg = inputs.PrefillConfig("inject", 2, 300, 8, 2, 64, dtype, top_k=6, window=40, seed=3)
    raw = inputs.make_prefill_inputs(cfg)
    q, k, v, g = _upload(cfg, raw)
    rng = np.random.default_rng(11)
    nb = -(-cfg.seqlen // cfg.block)
    inj = rng.integers(-2, nb + 2, size=(cfg.batch, cfg.seqlen, cfg.n_kv_heads, cfg.top_k)).astype(np.int32)
    inj[..., 1] = inj[..., 0]
    inj[..., 3] = inj[..., 2]
    inj[:, ::7] = -1                                        # some rows select nothing
    print(f"[prefill inject] {cfg}", flush=True)
    out = nsa.prefill(q, k, v, g, top_k=cfg.top_k, window=cfg.window, out_dtype=torch.float32,
                      idx=torch.from_numpy(inj).cuda(), inject=True)[0]
    torch.cuda.synchronize()
    orc = _oracle(cfg, raw, np.arange(cfg.seqlen), inject=inj)
    err = maxabs(out.cpu().numpy().astype(np.float64), orc["out"])
    assert err <= TOL[dtype], f"injected-selection error {err}"
