"""The allocation-free decode (nsa_fwd_decode_noalloc, the library's own
device scratch) against nsa_fwd_decode with a caller workspace: bit for bit,
on two calls in a row whose second is smaller, with the selection written to
idx and kept in the scratch."""

import numpy as np
import pytest
import torch

from long_context_sparse_fwd_amd import inputs, nsa
from tests.parity import dev

pytestmark = pytest.mark.gpu


def _tensors(cfg):
    raw = inputs.make_decode_inputs(cfg)
    q, kc, vc, g = (dev(raw[n], cfg.dtype) for n in ("q", "k_cache", "v_cache", "gates"))
    kb, vb = nsa.compress_kv(kc, vc)
    return q, kc, vc, kb, vb, torch.from_numpy(raw["seqlens"]).cuda(), g


def test_noalloc_decode_equals_decode_on_two_calls_the_second_smaller():
    # fp32 with D 128 over 8192 tokens keeps the compressed logits in the
    # scratch; the second, smaller call reuses the same scratch
    cases = [
        inputs.DecodeConfig("noalloc-big", 3, 8192, 16, 2, 128, "f32", top_k=6, window=300, seqlens=(8192, 5000, 77)),
        inputs.DecodeConfig("noalloc-small", 2, 1000, 16, 2, 128, "bf16", top_k=4, window=100, seqlens=(1000, 65)),
    ]
    for cfg in cases:
        print(f"[noalloc] {cfg.name}", flush=True)
        t = _tensors(cfg)
        ref, ref_idx = nsa.decode(*t, top_k=cfg.top_k, window=cfg.window, out_dtype=torch.float32, return_idx=True)
        out = torch.full_like(ref, float("nan"))
        idx = torch.full_like(ref_idx, -5)
        nsa.decode_noalloc(*t, top_k=cfg.top_k, window=cfg.window, out=out, idx=idx)
        out2 = torch.full_like(ref, float("nan"))
        nsa.decode_noalloc(*t, top_k=cfg.top_k, window=cfg.window, out=out2)   # the selection stays in the scratch
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), cfg.name
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), cfg.name
        assert torch.equal(out2.view(torch.int32), ref.view(torch.int32)), cfg.name
        assert np.isfinite(out.cpu().numpy()).all()
