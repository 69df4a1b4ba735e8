"""Seeded synthetic inputs for the NSA forward pass.

This module only draws and encodes data. It computes nothing of the attention
method itself, so the float64 oracle and the HIP path can both be fed from it
without sharing any of the method's arithmetic.

Recipe (stated once, used everywhere):

* Every tensor is built from 64-token chunks. Chunk ``(tensor_id, b, blk)`` is
  ``numpy.random.Generator(PCG64(SeedSequence([seed, tensor_id, b, blk])))
  .standard_normal(shape, dtype=float32)``. Tensor ids: 0 = Q, 1 = K, 2 = V,
  3 = gate logits, 4 = the upstream gradient of the output (backward pass).
  Chunk shapes are ``(64, Hq, D)``, ``(64, G, D)``, ``(64, G, D)``,
  ``(64, Hq, 3)`` and ``(64, Hq, D)``.
* Because the key never contains the sequence length, a shorter workload is an
  exact prefix of a longer one with the same seed and heads.
* bf16 values are the float32 draw rounded to nearest-even (stored as uint16
  bit patterns); fp32 values are the draw itself.
* Gates are ``sigmoid(logit)`` evaluated in float64, rounded to float32
  (nearest-even) and then, for bf16 workloads, to bf16 (nearest-even).
* Synthetic weights of the general geometry (no trained weights exist): the
  learned compressor ``wk``/``wv`` [D, block, D] is N(0,1) / (block *
  sqrt(D)) (so a compressed key has the spread of a block mean, 1/sqrt(block)
  per dimension) and ``bk``/``bv`` [D] is 0.1 N(0,1); the gate layer
  ``gate_w`` [Hq, D, 3] is N(0,1) / sqrt(D) and ``gate_b`` [Hq, 3] is N(0,1).
  Each tensor is one keyed draw ``(seed, tensor_id)``, ids 10..15, scaled in
  float32 and stored like the other inputs.
* Token-level sparse attention (DSA) adds, per 64-token chunk, the indexer
  queries ``qi`` (64, Hi, Di) drawn N(0,1) / sqrt(Di), the indexer keys ``ki``
  (64, Di) drawn N(0,1) and the indexer head weights ``w`` (64, Hi) drawn
  N(0,1) / sqrt(Hi) (tensor ids 20, 21, 22), so that a head's dot product is
  N(0,1) and a score has spread ~0.7; q, k, v follow the recipe above.
* Decode sequence ``b`` with length ``s`` is the prefill-shaped batch row ``b``
  read at position ``s - 1``: its query is row ``(s-1) % 64`` of Q chunk
  ``(0, b, (s-1)//64)``, its gates the same row of chunk ``(3, b, ...)``, and its
  K/V cache is made of K/V chunks ``(1|2, b, blk)`` laid out ``[B, G, Lmax, D]``.
  Cache positions at or beyond ``s`` hold ordinary draws that a correct kernel
  never reads into the result.

The workloads mirror the NSA how-to's ``[benchmark] seq_lengths`` (8192, 32768,
65536) and its ``[model.nsa]`` parameters (blocks of 64, top-k 16, window 512),
NSA how-to (qwbw.cn/news/106443), section 3 "config.toml skeleton".
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

TID_Q, TID_K, TID_V, TID_GATE, TID_DOUT = 0, 1, 2, 3, 4
# synthetic weights of the general geometry (one draw per tensor, not chunked)
TID_WK, TID_BK, TID_WV, TID_BV, TID_GW, TID_GB = 10, 11, 12, 13, 14, 15
# token-level sparse attention: indexer queries, indexer keys, indexer head weights
TID_QI, TID_KI, TID_WI = 20, 21, 22
CHUNK = 64


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    batch: int
    seqlen: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str  # "bf16" or "f32"
    top_k: int
    window: int
    block: int = 64
    seed: int = 0

    @property
    def kind(self) -> str:
        return "prefill"


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    max_seqlen: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    top_k: int
    window: int
    block: int = 64
    seed: int = 0
    # per-sequence lengths; None means every sequence is max_seqlen long
    seqlens: tuple | None = field(default=None)

    @property
    def kind(self) -> str:
        return "decode"

    def lengths(self) -> np.ndarray:
        if self.seqlens is None:
            return np.full(self.batch, self.max_seqlen, dtype=np.int32)
        assert len(self.seqlens) == self.batch
        return np.asarray(self.seqlens, dtype=np.int32)


# The five workloads: a tiny fp32 case, 8k / 32k / 64k bf16 prefill and a
# 64 x 64k bf16 decode.
CONFIGS = {
    "tiny": PrefillConfig("tiny", 1, 1024, 4, 1, 64, "f32", top_k=4, window=128),
    "p8k": PrefillConfig("p8k", 1, 8192, 64, 4, 128, "bf16", top_k=16, window=512),
    "p32k": PrefillConfig("p32k", 1, 32768, 64, 4, 128, "bf16", top_k=16, window=512),
    "p64k": PrefillConfig("p64k", 1, 65536, 64, 4, 128, "bf16", top_k=16, window=512),
    "d64k": DecodeConfig("d64k", 64, 65536, 64, 4, 128, "bf16", top_k=16, window=512),
}


@dataclass(frozen=True)
class DsaConfig:
    """Token-level sparse attention: indexer with idx_heads heads of idx_dim
    dimensions, top_k tokens per query; attention heads as in the prefill."""
    name: str
    batch: int
    seqlen: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    idx_heads: int
    idx_dim: int
    dtype: str
    top_k: int
    seed: int = 0

    @property
    def kind(self) -> str:
        return "dsa"


# The DSA how-to's prefill example: one 64K sequence, a 16-head indexer,
# top-k 2048, attention in the absorbed MLA form (one key/value head shared by
# all query heads); and a short case.
DSA_CONFIGS = {
    "dsa64k": DsaConfig("dsa64k", 1, 65536, 64, 1, 128, 16, 128, "bf16", top_k=2048),
    "dsa8k": DsaConfig("dsa8k", 1, 8192, 64, 1, 128, 16, 128, "bf16", top_k=2048),
}


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def chunk_normal(seed: int, tensor_id: int, b: int, blk: int, shape) -> np.ndarray:
    """Standard-normal float32 draw of one keyed 64-token chunk."""
    ss = np.random.SeedSequence([seed, tensor_id, b, blk])
    return np.random.Generator(np.random.PCG64(ss)).standard_normal(shape, dtype=np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns.

    Inputs are finite draws, so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 draw -> stored form (uint16 bits for bf16, float32 for f32)."""
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Stored form -> the exact same values as float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(stored).astype(np.float64)
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def gate_values(logits: np.ndarray, dtype: str) -> np.ndarray:
    """sigmoid(logit) in float64 -> float32 (RNE) -> stored dtype."""
    g = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
    return encode(g.astype(np.float32), dtype)


def storage_dtype(dtype: str):
    return np.uint16 if dtype == "bf16" else np.float32


def make_prefill_inputs(cfg: PrefillConfig, threads: int | None = None) -> dict:
    """Q [B,L,Hq,D], K/V [B,L,G,D], gates [B,L,Hq,3] in stored form."""
    B, L, Hq, G, D = cfg.batch, cfg.seqlen, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    sd = storage_dtype(cfg.dtype)
    out = {
        "q": np.empty((B, L, Hq, D), sd),
        "k": np.empty((B, L, G, D), sd),
        "v": np.empty((B, L, G, D), sd),
        "gates": np.empty((B, L, Hq, 3), sd),
    }
    nblk = (L + CHUNK - 1) // CHUNK

    def work(item):
        b, blk = item
        t0, t1 = blk * CHUNK, min(L, (blk + 1) * CHUNK)
        n = t1 - t0
        out["q"][b, t0:t1] = encode(chunk_normal(cfg.seed, TID_Q, b, blk, (CHUNK, Hq, D))[:n], cfg.dtype)
        out["k"][b, t0:t1] = encode(chunk_normal(cfg.seed, TID_K, b, blk, (CHUNK, G, D))[:n], cfg.dtype)
        out["v"][b, t0:t1] = encode(chunk_normal(cfg.seed, TID_V, b, blk, (CHUNK, G, D))[:n], cfg.dtype)
        out["gates"][b, t0:t1] = gate_values(
            chunk_normal(cfg.seed, TID_GATE, b, blk, (CHUNK, Hq, 3))[:n], cfg.dtype)

    items = [(b, blk) for b in range(B) for blk in range(nblk)]
    nw = threads or _workers()
    if nw == 1 or len(items) < 4:
        for it in items:
            work(it)
    else:
        with ThreadPoolExecutor(nw) as ex:
            list(ex.map(work, items))
    return out


def make_dout(cfg: PrefillConfig, dtype: str | None = None) -> np.ndarray:
    """Upstream gradient dout [B,L,Hq,D] in stored form (tensor id 4), in the
    output's dtype (the input dtype unless given)."""
    B, L, Hq, D = cfg.batch, cfg.seqlen, cfg.n_q_heads, cfg.head_dim
    dt = dtype or cfg.dtype
    out = np.empty((B, L, Hq, D), storage_dtype(dt))
    for b in range(B):
        for blk in range((L + CHUNK - 1) // CHUNK):
            t0, t1 = blk * CHUNK, min(L, (blk + 1) * CHUNK)
            out[b, t0:t1] = encode(chunk_normal(cfg.seed, TID_DOUT, b, blk, (CHUNK, Hq, D))[: t1 - t0], dt)
    return out


def _weight(seed: int, tensor_id: int, shape, scale: float, dtype: str) -> np.ndarray:
    ss = np.random.SeedSequence([seed, tensor_id])
    x = np.random.Generator(np.random.PCG64(ss)).standard_normal(shape, dtype=np.float32)
    return encode(x * np.float32(scale), dtype)


def make_compressor_weights(cfg: PrefillConfig, block: int) -> dict:
    """Synthetic learned compressor: wk, wv [D, block, D]; bk, bv [D] (stored form)."""
    D = cfg.head_dim
    ws = 1.0 / (block * np.sqrt(D))
    return {"wk": _weight(cfg.seed, TID_WK, (D, block, D), ws, cfg.dtype),
            "bk": _weight(cfg.seed, TID_BK, (D,), 0.1, cfg.dtype),
            "wv": _weight(cfg.seed, TID_WV, (D, block, D), ws, cfg.dtype),
            "bv": _weight(cfg.seed, TID_BV, (D,), 0.1, cfg.dtype)}


def make_gate_weights(cfg: PrefillConfig) -> dict:
    """Synthetic gate layer: gate_w [Hq, D, 3], gate_b [Hq, 3] (stored form)."""
    Hq, D = cfg.n_q_heads, cfg.head_dim
    return {"gate_w": _weight(cfg.seed, TID_GW, (Hq, D, 3), 1.0 / np.sqrt(D), cfg.dtype),
            "gate_b": _weight(cfg.seed, TID_GB, (Hq, 3), 1.0, cfg.dtype)}


def make_selection(cfg: PrefillConfig, share: int = 8) -> np.ndarray:
    """A seeded block selection idx [B,L,G,top_k] int32 in the forward's
    output form: each row holds the token's own block t // 64 and top_k - 1
    distinct earlier blocks drawn uniformly (all of them when there are fewer),
    ascending, padded with -1. The ``share`` consecutive tokens of an aligned
    group draw one set (their own block is the same). A stand-in selection for
    the backward pass, whose gradients take the selection as given."""
    B, L, G, n = cfg.batch, cfg.seqlen, cfg.n_kv_heads, cfg.top_k
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 5])))
    idx = np.full((B, L, G, n), -1, dtype=np.int32)
    for t0 in range(0, L, share):
        own = t0 // CHUNK
        m = min(n - 1, own)
        if m < own:
            pick = np.argpartition(rng.random((B, G, own)), m - 1, axis=2)[..., :m] if m > 0 else \
                np.zeros((B, G, 0), np.int64)
        else:
            pick = np.broadcast_to(np.arange(own), (B, G, own))
        rows = np.sort(np.concatenate([pick, np.full((B, G, 1), own)], axis=2), axis=2).astype(np.int32)
        idx[:, t0: t0 + share, :, : m + 1] = rows[:, None]
    return idx


def make_decode_inputs(cfg: DecodeConfig, threads: int | None = None) -> dict:
    """q [B,Hq,D], k/v cache [B,G,Lmax,D], gates [B,Hq,3], seqlens [B] int32."""
    B, Lm, Hq, G, D = cfg.batch, cfg.max_seqlen, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    sd = storage_dtype(cfg.dtype)
    lens = cfg.lengths()
    out = {
        "q": np.empty((B, Hq, D), sd),
        "k_cache": np.empty((B, G, Lm, D), sd),
        "v_cache": np.empty((B, G, Lm, D), sd),
        "gates": np.empty((B, Hq, 3), sd),
        "seqlens": lens.copy(),
    }
    for b in range(B):
        s = int(lens[b])
        pos = max(s, 1) - 1
        blk, r = divmod(pos, CHUNK)
        out["q"][b] = encode(chunk_normal(cfg.seed, TID_Q, b, blk, (CHUNK, Hq, D))[r], cfg.dtype)
        out["gates"][b] = gate_values(chunk_normal(cfg.seed, TID_GATE, b, blk, (CHUNK, Hq, 3))[r], cfg.dtype)

    nblk = (Lm + CHUNK - 1) // CHUNK

    def work(item):
        b, blk = item
        t0, t1 = blk * CHUNK, min(Lm, (blk + 1) * CHUNK)
        n = t1 - t0
        kk = chunk_normal(cfg.seed, TID_K, b, blk, (CHUNK, G, D))[:n]
        vv = chunk_normal(cfg.seed, TID_V, b, blk, (CHUNK, G, D))[:n]
        out["k_cache"][b, :, t0:t1] = encode(kk, cfg.dtype).transpose(1, 0, 2)
        out["v_cache"][b, :, t0:t1] = encode(vv, cfg.dtype).transpose(1, 0, 2)

    items = [(b, blk) for b in range(B) for blk in range(nblk)]
    nw = threads or _workers()
    if nw == 1 or len(items) < 4:
        for it in items:
            work(it)
    else:
        with ThreadPoolExecutor(nw) as ex:
            list(ex.map(work, items))
    return out


def make_dsa_inputs(cfg: DsaConfig, threads: int | None = None) -> dict:
    """q [B,L,Hq,D], k/v [B,L,G,D], qi [B,L,Hi,Di], ki [B,L,Di], w [B,L,Hi] in stored form."""
    B, L, Hq, G, D, Hi, Di = (cfg.batch, cfg.seqlen, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.idx_heads,
                              cfg.idx_dim)
    sd = storage_dtype(cfg.dtype)
    out = {
        "q": np.empty((B, L, Hq, D), sd),
        "k": np.empty((B, L, G, D), sd),
        "v": np.empty((B, L, G, D), sd),
        "qi": np.empty((B, L, Hi, Di), sd),
        "ki": np.empty((B, L, Di), sd),
        "w": np.empty((B, L, Hi), sd),
    }
    nblk = (L + CHUNK - 1) // CHUNK
    sq, sw = np.float32(1.0 / np.sqrt(Di)), np.float32(1.0 / np.sqrt(Hi))

    def work(item):
        b, blk = item
        t0, t1 = blk * CHUNK, min(L, (blk + 1) * CHUNK)
        n = t1 - t0
        out["q"][b, t0:t1] = encode(chunk_normal(cfg.seed, TID_Q, b, blk, (CHUNK, Hq, D))[:n], cfg.dtype)
        out["k"][b, t0:t1] = encode(chunk_normal(cfg.seed, TID_K, b, blk, (CHUNK, G, D))[:n], cfg.dtype)
        out["v"][b, t0:t1] = encode(chunk_normal(cfg.seed, TID_V, b, blk, (CHUNK, G, D))[:n], cfg.dtype)
        out["qi"][b, t0:t1] = encode(chunk_normal(cfg.seed, TID_QI, b, blk, (CHUNK, Hi, Di))[:n] * sq, cfg.dtype)
        out["ki"][b, t0:t1] = encode(chunk_normal(cfg.seed, TID_KI, b, blk, (CHUNK, Di))[:n], cfg.dtype)
        out["w"][b, t0:t1] = encode(chunk_normal(cfg.seed, TID_WI, b, blk, (CHUNK, Hi))[:n] * sw, cfg.dtype)

    items = [(b, blk) for b in range(B) for blk in range(nblk)]
    nw = threads or _workers()
    if nw == 1 or len(items) < 4:
        for it in items:
            work(it)
    else:
        with ThreadPoolExecutor(nw) as ex:
            list(ex.map(work, items))
    return out
