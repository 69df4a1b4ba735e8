"""GPU parity of nsa_fwd_decode and nsa_compress_kv against the float64 oracle."""

import numpy as np
import pytest
import torch

from long_context_sparse_fwd_amd import inputs, nsa
from oracle import nsa_ref
from tests.parity import TOL, Lazy, check_indices, dev, maxabs

pytestmark = pytest.mark.gpu


def _block_cache_f64(cache_f32: np.ndarray, block: int) -> np.ndarray:
    """Oracle block means of a [B, G, L, D] cache -> [B, G, L//block, D] float64."""
    return nsa_ref.compress(cache_f32.transpose(0, 2, 1, 3), block).transpose(0, 2, 1, 3)


def _stored(x64: np.ndarray, dtype: str) -> np.ndarray:
    return inputs.encode(x64.astype(np.float32), dtype)


def run_decode(cfg, batches=None, check_c=True):
    raw = inputs.make_decode_inputs(cfg)
    B = cfg.batch
    batches = list(range(B)) if batches is None else batches
    print(f"[decode] {cfg.name} B={B} Lmax={cfg.max_seqlen} batches={batches}", flush=True)
    q, kc_, vc_, g = (dev(raw[n], cfg.dtype) for n in ("q", "k_cache", "v_cache", "gates"))
    # block cache: the oracle's block means (stored in the input dtype) feed both
    # sides for the checked sequences; the others use the library's own means
    kbd, vbd = nsa.compress_kv(kc_, vc_)
    torch.cuda.synchronize()
    kb = np.zeros((B, cfg.n_kv_heads, cfg.max_seqlen // cfg.block, cfg.head_dim), raw["k_cache"].dtype)
    vb = np.zeros_like(kb)
    for b in batches:
        kb[b] = _stored(_block_cache_f64(Lazy(raw["k_cache"], cfg.dtype)[b:b + 1], cfg.block)[0], cfg.dtype)
        vb[b] = _stored(_block_cache_f64(Lazy(raw["v_cache"], cfg.dtype)[b:b + 1], cfg.block)[0], cfg.dtype)
        kbd[b] = dev(kb[b], cfg.dtype)
        vbd[b] = dev(vb[b], cfg.dtype)
    lens = torch.from_numpy(raw["seqlens"]).cuda()
    out, idx = nsa.decode(q, kc_, vc_, kbd, vbd, lens, g, top_k=cfg.top_k, window=cfg.window,
                          out_dtype=torch.float32, return_idx=True)
    torch.cuda.synchronize()
    go, gi = out.cpu().numpy().astype(np.float64), idx.cpu().numpy()

    sel = np.asarray(batches)
    lz = lambda n: Lazy(raw[n], cfg.dtype)
    sub = lambda n: lz(n)[sel]
    orc = nsa_ref.decode(sub("q"), sub("k_cache"), sub("v_cache"), Lazy(kb, cfg.dtype)[sel],
                         Lazy(vb, cfg.dtype)[sel], raw["seqlens"][sel], sub("gates"), block=cfg.block,
                         top_k=cfg.top_k, window=cfg.window)
    n = cfg.top_k
    own = np.broadcast_to(((raw["seqlens"][sel] - 1) // cfg.block)[:, None], orc["idx"].shape[:2])
    sc = orc["scores"]
    sc = sc.reshape(-1, sc.shape[-1]) if sc.shape[-1] else np.zeros((own.size, 1))
    exact, excused, bad = check_indices(gi[sel].reshape(-1, n), orc["idx"].reshape(-1, n),
                                        orc["gap"].reshape(-1), sc, own.reshape(-1), n)
    assert not bad, f"index mismatches: {bad[:5]}"
    expect = orc["out"].copy()
    for r in np.argwhere(np.any(gi[sel] != orc["idx"], axis=2))[:, 0]:
        b = sel[r]
        re = nsa_ref.decode(lz("q")[b:b + 1], lz("k_cache")[b:b + 1], lz("v_cache")[b:b + 1],
                            Lazy(kb, cfg.dtype)[b:b + 1], Lazy(vb, cfg.dtype)[b:b + 1],
                            raw["seqlens"][b:b + 1], lz("gates")[b:b + 1], block=cfg.block,
                            top_k=n, window=cfg.window, inject_idx=gi[b:b + 1])
        expect[r] = re["out"][0]
    err_b = maxabs(go[sel], expect)
    assert err_b <= TOL[cfg.dtype], f"decode output error {err_b}"
    err_c = None
    if check_c:
        inj = gi.copy()
        inj[sel] = orc["idx"]
        oc = nsa.decode(q, kc_, vc_, kbd, vbd, lens, g, top_k=n, window=cfg.window,
                        out_dtype=torch.float32, idx=torch.from_numpy(inj).cuda(), inject=True)[0]
        torch.cuda.synchronize()
        err_c = maxabs(oc.cpu().numpy()[sel], orc["out"])
        assert err_c <= TOL[cfg.dtype], f"decode injected-index error {err_c}"
    err_b16 = None
    if cfg.dtype == "bf16":
        # the benchmarked instance: bf16 output, the same fp32 result rounded once
        o16, i16 = nsa.decode(q, kc_, vc_, kbd, vbd, lens, g, top_k=cfg.top_k, window=cfg.window,
                              out_dtype=torch.bfloat16, return_idx=True)
        torch.cuda.synchronize()
        assert torch.equal(i16, idx), "the selection depends on the output type"
        assert torch.equal(o16.view(torch.int16), out.to(torch.bfloat16).view(torch.int16))
        err_b16 = maxabs(o16.float().cpu().numpy().astype(np.float64)[sel], expect)
        assert err_b16 <= TOL["bf16"], f"decode bf16-output error {err_b16}"
    print(f"  exact={exact} excused={excused} errB={err_b:.3g} errC={err_c} bf16-out errB={err_b16}", flush=True)
    return {"raw": raw, "gpu_out": go, "gpu_idx": gi, "dev": (q, kc_, vc_, kbd, vbd, lens, g)}


@pytest.mark.parametrize("cfg", [
    inputs.DecodeConfig("dec-mixed", 6, 1000, 16, 2, 128, "bf16", top_k=7, window=130,
                        seqlens=(1, 63, 64, 700, 1000, 129)),
    inputs.DecodeConfig("dec-f32", 3, 700, 8, 2, 64, "f32", top_k=4, window=64, seqlens=(700, 65, 333)),
    # fp32 with D 128: logits in LDS, no room to park the window states
    inputs.DecodeConfig("dec-f32-d128", 2, 900, 8, 2, 128, "f32", top_k=5, window=200, seqlens=(900, 321)),
    # fp32 with D 128 and 128 blocks: the compressed logits go to the workspace
    inputs.DecodeConfig("dec-f32-d128-long", 2, 8192, 8, 1, 128, "f32", top_k=6, window=300,
                        seqlens=(8192, 5000)),
    inputs.DecodeConfig("dec-bf16-long", 2, 8192, 64, 4, 128, "bf16", top_k=16, window=512),
    # bf16 with D 64 and 512 blocks: the window states are parked in the logits region
    inputs.DecodeConfig("dec-bf16-d64-park", 2, 32768, 16, 1, 64, "bf16", top_k=8, window=256,
                        seqlens=(32768, 30001)),
    inputs.DecodeConfig("dec-window-all", 2, 300, 4, 1, 64, "bf16", top_k=2, window=5000,
                        seqlens=(300, 190)),
], ids=lambda c: c.name)
def test_decode_matches_oracle(cfg):
    run_decode(cfg)


def test_decode_full_size_d64k_sampled():
    # every fourth sequence, plus two odd ones: 18 of the 64
    rep = run_decode(inputs.CONFIGS["d64k"], batches=sorted(set(range(0, 64, 4)) | {17, 63}), check_c=True)
    gi = rep["gpu_idx"]
    own = 1023
    assert np.all(gi[:, :, -1] == own)          # ascending with the own block last
    assert np.all(np.diff(gi, axis=-1) > 0)
    assert np.all(np.isfinite(rep["gpu_out"]))


def test_invalid_seqlens_give_zero_output_and_no_selection():
    cfg = inputs.DecodeConfig("dec-bad", 3, 256, 16, 1, 64, "bf16", top_k=3, window=40,
                              seqlens=(100, 256, 50))
    raw = inputs.make_decode_inputs(cfg)
    q, kc_, vc_, g = (dev(raw[n], "bf16") for n in ("q", "k_cache", "v_cache", "gates"))
    kb, vb = nsa.compress_kv(kc_, vc_)
    lens = torch.tensor([0, 257, 50], dtype=torch.int32, device="cuda")
    out, idx = nsa.decode(q, kc_, vc_, kb, vb, lens, g, top_k=3, window=40, out_dtype=torch.float32,
                          return_idx=True)
    torch.cuda.synchronize()
    assert torch.all(out[:2] == 0) and torch.all(idx[:2] == -1)
    assert torch.all(torch.isfinite(out[2])) and torch.any(out[2] != 0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_compress_kv_matches_oracle_block_means(dtype):
    cfg = inputs.DecodeConfig("cmp", 2, 64 * 9 + 17, 4, 3, 128, dtype, top_k=2, window=8)
    raw = inputs.make_decode_inputs(cfg)
    k, v = dev(raw["k_cache"], dtype), dev(raw["v_cache"], dtype)
    kc, vc = nsa.compress_kv(k, v)
    torch.cuda.synchronize()
    assert kc.shape == (2, 3, 9, 128)
    for got, name in ((kc, "k_cache"), (vc, "v_cache")):
        ref = _block_cache_f64(Lazy(raw[name], dtype)[:], 64)
        err = np.abs(got.float().cpu().numpy() - ref)
        # one rounding of an fp32 sum of 64 values
        bound = (2.0 ** -8 if dtype == "bf16" else 2.0 ** -20) * np.abs(ref) + 1e-6
        assert np.all(err <= bound), float(err.max())


def test_decode_equals_prefill_last_rows_on_gpu():
    # decode of sequence b at length s reproduces prefill row s-1 of the same data
    L, G, Hq, D = 1500, 4, 64, 128
    pcfg = inputs.PrefillConfig("pd", 2, L, Hq, G, D, "bf16", top_k=16, window=512)
    raw = inputs.make_prefill_inputs(pcfg)
    q, k, v, g = (dev(raw[n], "bf16") for n in ("q", "k", "v", "gates"))
    pout, pidx = nsa.prefill(q, k, v, g, top_k=16, window=512, out_dtype=torch.float32, return_idx=True)
    lens = torch.tensor([L, 1000], dtype=torch.int32, device="cuda")
    kcache = k.transpose(1, 2).contiguous()
    vcache = v.transpose(1, 2).contiguous()
    kb, vb = nsa.compress_kv(kcache, vcache)
    qd = torch.stack([q[0, L - 1], q[1, 999]])
    gd = torch.stack([g[0, L - 1], g[1, 999]])
    dout, didx = nsa.decode(qd, kcache, vcache, kb, vb, lens, gd, top_k=16, window=512,
                            out_dtype=torch.float32, return_idx=True)
    torch.cuda.synchronize()
    rows = [(0, L - 1), (1, 999)]
    for i, (b, t) in enumerate(rows):
        same = torch.equal(didx[i], pidx[b, t])
        err = (dout[i] - pout[b, t]).abs().max().item()
        # identical block means and products; only summation orders differ
        assert err <= (1e-3 if same else 2e-1), (i, same, err)


def test_decode_injected_selection_with_repeats_and_unusable_entries():
    cfg = inputs.DecodeConfig("dec-inject", 4, 700, 8, 2, 64, "bf16", top_k=6, window=100,
                              seqlens=(700, 65, 333, 1))
    raw = inputs.make_decode_inputs(cfg)
    print(f"[decode inject] {cfg.name}", flush=True)
    q, kc_, vc_, g = (dev(raw[n], cfg.dtype) for n in ("q", "k_cache", "v_cache", "gates"))
    kb = _stored(_block_cache_f64(Lazy(raw["k_cache"], cfg.dtype)[:], cfg.block), cfg.dtype)
    vb = _stored(_block_cache_f64(Lazy(raw["v_cache"], cfg.dtype)[:], cfg.block), cfg.dtype)
    kbd, vbd = dev(kb, cfg.dtype), dev(vb, cfg.dtype)
    lens = torch.from_numpy(raw["seqlens"]).cuda()
    rng = np.random.default_rng(13)
    nb = cfg.max_seqlen // cfg.block
    inj = rng.integers(-2, nb + 2, size=(cfg.batch, cfg.n_kv_heads, cfg.top_k)).astype(np.int32)
    inj[..., 1] = inj[..., 0]
    inj[2, 1] = -1                                          # one (sequence, group) selects nothing
    out = nsa.decode(q, kc_, vc_, kbd, vbd, lens, g, top_k=cfg.top_k, window=cfg.window,
                     out_dtype=torch.float32, idx=torch.from_numpy(inj).cuda(), inject=True)[0]
    torch.cuda.synchronize()
    lz = lambda n: Lazy(raw[n], cfg.dtype)
    orc = nsa_ref.decode(lz("q")[:], lz("k_cache")[:], lz("v_cache")[:], Lazy(kb, cfg.dtype)[:],
                         Lazy(vb, cfg.dtype)[:], raw["seqlens"], lz("gates")[:], block=cfg.block,
                         top_k=cfg.top_k, window=cfg.window, inject_idx=inj)
    err = maxabs(out.cpu().numpy().astype(np.float64), orc["out"])
    assert err <= TOL[cfg.dtype], f"decode injected-selection error {err}"


def test_decode_is_deterministic():
    """The merges combine the waves' states in a fixed order: repeated calls agree bit for bit."""
    cfg = inputs.DecodeConfig("dec-det", 4, 4096, 32, 2, 128, "bf16", top_k=16, window=512,
                              seqlens=(4096, 4000, 2049, 777))
    raw = inputs.make_decode_inputs(cfg)
    q, kc_, vc_, g = (dev(raw[n], cfg.dtype) for n in ("q", "k_cache", "v_cache", "gates"))
    kb, vb = nsa.compress_kv(kc_, vc_)
    lens = torch.from_numpy(raw["seqlens"]).cuda()
    runs = [nsa.decode(q, kc_, vc_, kb, vb, lens, g, top_k=cfg.top_k, window=cfg.window, return_idx=True)
            for _ in range(10)]
    torch.cuda.synchronize()
    for o, i in runs[1:]:
        assert torch.equal(o.view(torch.int16), runs[0][0].view(torch.int16))
        assert torch.equal(i, runs[0][1])
