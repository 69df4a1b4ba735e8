"""Every entry point writes only its outputs and its workspace.

Outputs, selections, gradients and workspaces are views into larger device
buffers whose surroundings hold a sentinel; after each call the sentinel
must be intact on both sides, and each result must equal the same call made
with plain tensors (so the views were really used). Covers the plain and
general prefill, the decode, token-level sparse attention and the backward
pass, with bf16 outputs where the benchmark times them.
"""

import numpy as np
import pytest
import torch

from long_context_sparse_fwd_amd import inputs, nsa
from tests.parity import dev

pytestmark = pytest.mark.gpu

GUARD = 1 << 16          # bytes of sentinel on each side
BYTE = 0xA5


class Guarded:
    """A tensor of `shape`/`dtype` inside a buffer with GUARD sentinel bytes on each side."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((GUARD + n + GUARD,), BYTE, dtype=torch.uint8, device="cuda")
        self.n = n
        self.t = self.buf[GUARD:GUARD + n].view(dtype).view(*shape)

    def intact(self) -> bool:
        torch.cuda.synchronize()
        return bool(torch.all(self.buf[:GUARD] == BYTE)) and bool(torch.all(self.buf[GUARD + self.n:] == BYTE))


def _ws(nbytes):
    return Guarded((max(nbytes, 1),), torch.uint8)


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def test_prefill_outputs_and_workspace_stay_in_bounds():
    cfg = inputs.PrefillConfig("guard", 2, 777, 16, 2, 128, "bf16", top_k=8, window=100)
    raw = inputs.make_prefill_inputs(cfg)
    q, k, v, g = (dev(raw[n], cfg.dtype) for n in ("q", "k", "v", "gates"))
    ref, ridx = nsa.prefill(q, k, v, g, top_k=8, window=100, out_dtype=torch.bfloat16, return_idx=True)
    out = Guarded((2, 777, 16, 128), torch.bfloat16)
    idx = Guarded((2, 777, 2, 8), torch.int32)
    ws = _ws(nsa.prefill_workspace_bytes(q, k, v, g, out.t, top_k=8, window=100))
    nsa.prefill(q, k, v, g, top_k=8, window=100, out=out.t, idx=idx.t, workspace=ws.t)
    assert out.intact() and idx.intact() and ws.intact()
    assert _same(out.t, ref) and _same(idx.t, ridx)


def test_general_prefill_outputs_and_workspace_stay_in_bounds():
    cfg = inputs.PrefillConfig("guard-general", 1, 700, 16, 2, 128, "bf16", top_k=8, window=128, seed=3)
    raw = inputs.make_prefill_inputs(cfg)
    q, k, v = (dev(raw[n], cfg.dtype) for n in ("q", "k", "v"))
    W = inputs.make_compressor_weights(cfg, 32)
    GW = inputs.make_gate_weights(cfg)
    comp = tuple(dev(W[n], cfg.dtype) for n in ("wk", "bk", "wv", "bv"))
    gl = tuple(dev(GW[n], cfg.dtype) for n in ("gate_w", "gate_b"))
    kw = dict(top_k=8, window=128, block=32, select_block=64, stride=16, compressor=comp, gate_layer=gl)
    ref, ridx = nsa.prefill_general(q, k, v, None, out_dtype=torch.bfloat16, return_idx=True, **kw)
    out = Guarded((1, 700, 16, 128), torch.bfloat16)
    idx = Guarded((1, 700, 2, 8), torch.int32)
    nb = nsa.prefill_general_workspace_bytes(q, k, v, None, out.t, **kw)
    ws = _ws(nb)
    nsa.prefill_general(q, k, v, None, out=out.t, idx=idx.t, workspace=ws.t, **kw)
    assert out.intact() and idx.intact() and ws.intact()
    assert _same(out.t, ref) and _same(idx.t, ridx)


def test_decode_outputs_and_workspace_stay_in_bounds():
    cfg = inputs.DecodeConfig("guard-decode", 6, 2048, 16, 2, 128, "bf16", top_k=8, window=200,
                              seqlens=(2048, 1, 63, 64, 1500, 0))
    raw = inputs.make_decode_inputs(cfg)
    q, kc, vc, g = (dev(raw[n], cfg.dtype) for n in ("q", "k_cache", "v_cache", "gates"))
    kb, vb = nsa.compress_kv(kc, vc)
    lens = torch.from_numpy(raw["seqlens"]).cuda()
    ref, ridx = nsa.decode(q, kc, vc, kb, vb, lens, g, top_k=8, window=200, out_dtype=torch.bfloat16,
                           return_idx=True)
    out = Guarded((6, 16, 128), torch.bfloat16)
    idx = Guarded((6, 2, 8), torch.int32)
    ws = _ws(nsa.decode_workspace_bytes(q, kc, vc, kb, vb, g, out.t, top_k=8, window=200))
    nsa.decode(q, kc, vc, kb, vb, lens, g, top_k=8, window=200, out=out.t, idx=idx.t, workspace=ws.t)
    assert out.intact() and idx.intact() and ws.intact()
    assert _same(out.t, ref) and _same(idx.t, ridx)


def test_dsa_outputs_and_workspace_stay_in_bounds():
    cfg = inputs.DsaConfig("guard-dsa", 2, 1500, 16, 1, 128, 16, 128, "bf16", top_k=256, seed=4)
    raw = inputs.make_dsa_inputs(cfg)
    ts = [dev(raw[n], cfg.dtype) for n in ("q", "k", "v", "qi", "ki", "w")]
    ref, ridx = nsa.dsa_prefill(*ts, top_k=256, out_dtype=torch.bfloat16, return_idx=True)
    out = Guarded((2, 1500, 16, 128), torch.bfloat16)
    idx = Guarded((2, 1500, 256), torch.int32)
    ws = _ws(nsa.dsa_workspace_bytes(*ts, out.t, top_k=256))
    nsa.dsa_prefill(*ts, top_k=256, out=out.t, idx=idx.t, workspace=ws.t)
    assert out.intact() and idx.intact() and ws.intact()
    assert _same(out.t, ref) and _same(idx.t, ridx)


def test_backward_gradients_and_workspace_stay_in_bounds():
    cfg = inputs.PrefillConfig("guard-bwd", 1, 500, 16, 2, 128, "bf16", top_k=4, window=80, seed=5)
    raw = inputs.make_prefill_inputs(cfg)
    q, k, v, g = (dev(raw[n], cfg.dtype) for n in ("q", "k", "v", "gates"))
    out, idx = nsa.prefill(q, k, v, g, top_k=4, window=80, return_idx=True)
    dout = torch.randn(out.shape, generator=torch.Generator().manual_seed(6)).to(torch.bfloat16).cuda()
    # dk and dv come from float atomics, so two runs may differ in the last
    # bits: compare with a tolerance, and the guards exactly
    ref = nsa.prefill_backward(q, k, v, g, dout, idx, top_k=4, window=80)
    shapes = [(1, 500, 16, 128), (1, 500, 2, 128), (1, 500, 2, 128), (1, 500, 16, 3)]
    gr = [Guarded(s, torch.float32) for s in shapes]
    ws = _ws(nsa.prefill_backward_workspace_bytes(q, k, v, g, dout, top_k=4, window=80))
    nsa.prefill_backward(q, k, v, g, dout, idx, top_k=4, window=80, grads=tuple(x.t for x in gr), workspace=ws.t)
    assert ws.intact() and all(x.intact() for x in gr)
    for got, want in zip(gr, ref):
        assert torch.allclose(got.t, want, rtol=1e-5, atol=1e-6)
