"""GPU parity of nsa_fwd_decode_general (the decode with the general
geometry) against the float64 oracle's decode, through the C ABI: a
compression stride below the block size (overlapping compressed blocks, given
as a block cache), selection blocks larger than the compressed blocks
(including sizes that are not a multiple of 64) and a gate layer with seeded
synthetic weights. Checks A, B and C as for the plain decode, on fp32 and
bf16 output; the general entry with the plain geometry must reproduce
nsa_fwd_decode bit for bit.
"""

import numpy as np
import pytest
import torch

from long_context_sparse_fwd_amd import inputs, nsa
from oracle import nsa_ref
from tests.parity import TOL, Lazy, check_indices, dev, maxabs

pytestmark = pytest.mark.gpu


def _cache_f64(cache: np.ndarray, block: int, stride: int) -> np.ndarray:
    """Oracle block means [B, G, Nc, D] of the blocks [i*stride, i*stride + block) of a [B, G, L, D] cache."""
    return nsa_ref.compress(cache.transpose(0, 2, 1, 3), block, stride).transpose(0, 2, 1, 3)


def run_decode_general(cfg, l, d, ls, gate_layer=False, check_c=True):
    raw = inputs.make_decode_inputs(cfg)
    print(f"[decode general] {cfg.name} l={l} d={d} l'={ls} gate_layer={gate_layer}", flush=True)
    q, kc_, vc_, g = (dev(raw[n], cfg.dtype) for n in ("q", "k_cache", "v_cache", "gates"))
    lz = lambda n: Lazy(raw[n], cfg.dtype)
    kb = inputs.encode(_cache_f64(lz("k_cache")[:], l, d).astype(np.float32), cfg.dtype)
    vb = inputs.encode(_cache_f64(lz("v_cache")[:], l, d).astype(np.float32), cfg.dtype)
    kbd, vbd = dev(kb, cfg.dtype), dev(vb, cfg.dtype)
    lens = torch.from_numpy(raw["seqlens"]).cuda()
    if gate_layer:
        GW = inputs.make_gate_weights(cfg)
        gl = tuple(dev(GW[n], cfg.dtype) for n in ("gate_w", "gate_b"))
        gates_o = nsa_ref.gates_from_query(inputs.to_f64(raw["q"], cfg.dtype)[:, None],
                                           inputs.to_f64(GW["gate_w"], cfg.dtype),
                                           inputs.to_f64(GW["gate_b"], cfg.dtype))[:, 0]
    else:
        gl, gates_o = None, lz("gates")[:]

    def call(out_dtype, idx=None, inject=False, return_idx=False):
        return nsa.decode_general(q, kc_, vc_, kbd, vbd, lens, None if gate_layer else g, top_k=cfg.top_k,
                                  window=cfg.window, block=l, select_block=ls, stride=d, gate_layer=gl,
                                  out_dtype=out_dtype, idx=idx, inject=inject, return_idx=return_idx)

    def oracle(inject=None, bsl=slice(None)):
        return nsa_ref.decode(lz("q")[bsl], lz("k_cache")[bsl], lz("v_cache")[bsl], Lazy(kb, cfg.dtype)[bsl],
                              Lazy(vb, cfg.dtype)[bsl], raw["seqlens"][bsl], gates_o[bsl], block=l,
                              select_block=ls, stride=d, top_k=cfg.top_k, window=cfg.window, inject_idx=inject)

    out, idx = call(torch.float32, return_idx=True)
    torch.cuda.synchronize()
    go, gi = out.cpu().numpy().astype(np.float64), idx.cpu().numpy()
    orc = oracle()
    n = cfg.top_k
    own = np.broadcast_to(((raw["seqlens"] - 1) // ls)[:, None], orc["idx"].shape[:2])
    sc = orc["scores"]
    exact, excused, bad = check_indices(gi.reshape(-1, n), orc["idx"].reshape(-1, n), orc["gap"].reshape(-1),
                                        sc.reshape(-1, sc.shape[-1]), own.reshape(-1), n)
    assert not bad, f"index mismatches: {bad[:5]}"
    expect = orc["out"].copy()
    for b in np.argwhere(np.any(gi != orc["idx"], axis=2))[:, 0]:
        expect[b] = oracle(inject=gi[b:b + 1], bsl=slice(b, b + 1))["out"][0]
    err_b = maxabs(go, expect)
    assert err_b <= TOL[cfg.dtype], f"decode output error {err_b}"
    err_c = None
    if check_c:
        oc = call(torch.float32, idx=torch.from_numpy(orc["idx"].astype(np.int32)).cuda(), inject=True)[0]
        torch.cuda.synchronize()
        err_c = maxabs(oc.cpu().numpy().astype(np.float64), orc["out"])
        assert err_c <= TOL[cfg.dtype], f"decode injected-index error {err_c}"
    err_b16 = None
    if cfg.dtype == "bf16":
        o16, i16 = call(torch.bfloat16, return_idx=True)
        torch.cuda.synchronize()
        assert torch.equal(i16, idx), "the selection depends on the output type"
        assert torch.equal(o16.view(torch.int16), out.to(torch.bfloat16).view(torch.int16))
        err_b16 = maxabs(o16.float().cpu().numpy().astype(np.float64), expect)
        assert err_b16 <= TOL["bf16"], f"decode bf16-output error {err_b16}"
    print(f"  exact={exact} excused={excused} errB={err_b:.3g} errC={err_c} bf16-out errB={err_b16}", flush=True)


GEOMETRIES = [
    # name, config, l, d, l', gate layer
    ("overlap-d32", inputs.DecodeConfig("dg-overlap", 4, 2000, 16, 2, 128, "bf16", top_k=6, window=200,
                                        seqlens=(2000, 1, 95, 1337)), 64, 32, 64, False),
    ("select-128", inputs.DecodeConfig("dg-sel128", 3, 3000, 16, 2, 128, "bf16", top_k=8, window=300,
                                       seqlens=(3000, 200, 2049)), 64, 64, 128, False),
    ("l32-d16-ls96", inputs.DecodeConfig("dg-odd", 3, 1500, 8, 2, 64, "f32", top_k=5, window=100,
                                         seqlens=(1500, 96, 777)), 32, 16, 96, False),
    ("gate-layer", inputs.DecodeConfig("dg-gates", 3, 1200, 16, 1, 128, "bf16", top_k=4, window=150,
                                       seqlens=(1200, 64, 500)), 64, 64, 64, True),
    ("overlap-gates-f32", inputs.DecodeConfig("dg-og-f32", 2, 900, 8, 2, 64, "f32", top_k=6, window=64,
                                              seqlens=(900, 333)), 32, 8, 64, True),
    # 8192 tokens with blocks of 32 at stride 16: 511 compressed blocks
    ("long-bf16", inputs.DecodeConfig("dg-long", 2, 8192, 64, 4, 128, "bf16", top_k=16, window=512,
                                      seqlens=(8192, 6001)), 32, 16, 128, False),
    # 32768 tokens at stride 16: 2047 compressed blocks, logits in the workspace
    ("logits-in-workspace", inputs.DecodeConfig("dg-ws", 2, 32768, 16, 1, 64, "bf16", top_k=8, window=256,
                                                seqlens=(32768, 20000)), 32, 16, 64, False),
]


@pytest.mark.parametrize("case", GEOMETRIES, ids=[c[0] for c in GEOMETRIES])
def test_general_decode_matches_oracle(case):
    _, cfg, l, d, ls, gate_layer = case
    run_decode_general(cfg, l, d, ls, gate_layer=gate_layer)


def test_general_decode_with_the_plain_geometry_is_the_plain_decode():
    cfg = inputs.DecodeConfig("dg-plain", 3, 4000, 64, 4, 128, "bf16", top_k=16, window=512,
                              seqlens=(4000, 63, 2500))
    raw = inputs.make_decode_inputs(cfg)
    q, kc_, vc_, g = (dev(raw[n], cfg.dtype) for n in ("q", "k_cache", "v_cache", "gates"))
    kbd, vbd = nsa.compress_kv(kc_, vc_)
    lens = torch.from_numpy(raw["seqlens"]).cuda()
    o1, i1 = nsa.decode(q, kc_, vc_, kbd, vbd, lens, g, top_k=16, window=512, return_idx=True)
    o2, i2 = nsa.decode_general(q, kc_, vc_, kbd, vbd, lens, g, top_k=16, window=512, return_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
