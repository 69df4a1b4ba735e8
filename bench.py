#!/usr/bin/env python3
"""NSA forward benchmark on one MI355X (gfx950).

One step = one nsa_fwd_prefill call over the 64k workload (batch 1, 65536
tokens, 64 query heads in 4 KV groups, head_dim 128, blocks of 64, top-k 16,
window 512; bf16), the pages' 64k setting (NSA how-to, qwbw.cn/news/106443,
section 3). Inputs are seeded synthetic tensors already resident in HBM.

Prints ONE JSON line: tokens/s for prefill (the headline value), a roofline
object for the dominant kernel (algorithmic FLOPs over its HIP-event-timed
duration against the bf16 dense MFMA peak), the decode workload (64
sequences x 65536-token cache) as achieved HBM bandwidth, and the float64
CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
PREFILL_STAGES = ["k_prep", "k_cmpwin", "k_sel"]
BACKWARD_STAGES = ["prep", "query_side", "key_side"]
DECODE_STAGES = ["k_dec"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- algorithmic work

def pair_counts(L: int, block: int, top_k: int, window: int):
    """(query, key) pairs per head of one sequence for each branch, from the
    causal definitions: compressed floor((t+1)/l); selected the own block's
    t mod l + 1 tokens plus min(n-1, t//l) full earlier blocks; window
    min(t+1, w)."""
    t = np.arange(L, dtype=np.int64)
    cmp = int(((t + 1) // block).sum())
    slc = int(((t % block) + 1 + block * np.minimum(top_k - 1, t // block)).sum())
    win = int(np.minimum(t + 1, window).sum())
    return cmp, slc, win


def prefill_flops(cfg):
    cmp, slc, win = pair_counts(cfg.seqlen, cfg.block, cfg.top_k, cfg.window)
    per_pair = cfg.batch * cfg.n_q_heads * 4 * cfg.head_dim  # QK^T + PV
    return {"cmp": cmp * per_pair, "slc": slc * per_pair, "win": win * per_pair}


def decode_unique_bytes(cfg, idx: np.ndarray, lens: np.ndarray, cl=None, cd=None, ls=None) -> int:
    """Bytes the decode step must touch: block cache (the visible compressed
    blocks [i*cd, i*cd + cl)), selected blocks of ls tokens (tokens inside the
    window counted once), window, q, gates, out, idx."""
    cl = cl or cfg.block
    cd = cd or cl
    ls = ls or cfg.block
    D, G, Hq, el = cfg.head_dim, cfg.n_kv_heads, cfg.n_q_heads, 2
    total = 0
    for b in range(cfg.batch):
        s = int(lens[b])
        t = s - 1
        wlo = max(0, s - cfg.window)
        nvis = (s - cl) // cd + 1 if s >= cl else 0
        for g in range(G):
            toks = set(range(wlo, s))
            for j in idx[b, g]:
                if 0 <= j <= t // ls:
                    toks.update(range(j * ls, min(j * ls + ls, s)))
            total += (nvis * D * 2 + len(toks) * D * 2) * el
        total += Hq * D * el * 2 + Hq * 3 * el + G * cfg.top_k * 4
    return total


# ---------------------------------------------------------------- HIP events

class HipEvents:
    """hipEvent_t handles from the HIP runtime already loaded by torch."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e)
        self.arr = (ctypes.c_void_p * n)(*[e.value for e in self.ev])

    def array(self, first: int, count: int):
        return ctypes.cast(ctypes.byref(self.arr, first * ctypes.sizeof(ctypes.c_void_p)),
                           ctypes.POINTER(ctypes.c_void_p))

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


# ---------------------------------------------------------------- traffic from committed counters

# the sources each family of forward kernels (and their launches) is built from
DIGEST_SOURCES = {
    "nsa": ("nsa_api.cpp", "nsa_compress.hip", "nsa_decode.hip", "nsa_device.h", "nsa_internal.h",
            "nsa_prefill.hip", "nsa_topk.h"),
    "dsa": ("nsa_api.cpp", "nsa_device.h", "nsa_dsa.hip", "nsa_internal.h"),
}


def kernel_source_digest(family: str = "nsa") -> str:
    """Digest of the sources a family of forward kernels is built from
    (DIGEST_SOURCES); a committed counter record applies while it matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "long_context_sparse_fwd_amd", "csrc")
    for name in DIGEST_SOURCES[family]:
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def probe_gather_ceiling():
    """TB/s of random 16 KiB half-block reads from a 32 MiB per-XCD working
    set (the selected branch's pattern at 64k), as committed from the
    gather probe (best of its in-flight depths); None if absent."""
    path = os.path.join(ROOT, "profiles", "gather_ceiling_random_halfblocks.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"^\| 32 MiB[^|]*\|([^\n]*)$", open(path).read(), re.M)
    if not m:
        return None
    vals = [float(x) for x in re.findall(r"([0-9]+\.[0-9]+)", m.group(1))]
    return max(vals) if vals else None


def committed_traffic(kernel: str, workload: str, family: str = "nsa"):
    """HBM bytes per launch recorded from rocprofv3 FETCH_SIZE/WRITE_SIZE runs,
    if taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"pmc_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_digest:\s*(\w+)", text)
    if not m or m.group(1) != kernel_source_digest(family):
        return None
    m = re.search(rf"traffic_bytes_per_launch\s+{kernel}:\s*([0-9.eE+]+)", text)
    return float(m.group(1)) if m else None


# ---------------------------------------------------------------- CPU oracle baseline

class _LazyBf16:
    def __init__(self, arr):
        self.arr, self.shape = arr, arr.shape

    def __getitem__(self, key):
        from long_context_sparse_fwd_amd import inputs
        return inputs.bf16_bits_to_f32(self.arr[key])


def host_description():
    """CPU model (from /proc/cpuinfo) and the BLAS library numpy calls."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer')})"
                for i in threadpool_info() if i.get("user_api") == "blas"]
        blas = "; ".join(libs) or None
    except Exception:
        pass
    if blas is None:
        try:
            cfg = np.show_config(mode="dicts")
            b = cfg.get("Build Dependencies", {}).get("blas", {})
            blas = f"{b.get('name')} {b.get('version')}"
        except Exception:
            blas = "unknown"
    return model or "unknown", blas


def cpu_baseline(cfg, raw, seconds: float, gpu=None):
    """The float64 oracle on evenly spaced query rows of the same workload.

    With gpu = (out, idx) from the library on the same input (bf16 output,
    as timed), the oracle rows just computed also give the parity of that
    output: the selection compared row by row, and the largest absolute
    output error against the oracle run with the library's own selection
    where the two differ (the tests' Check B)."""
    from oracle import nsa_ref
    try:
        ncores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        ncores = os.cpu_count() or 1
    cpu_model, blas = host_description()
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=ncores)
    except Exception:  # pragma: no cover
        limiter = None
    lz = {n: _LazyBf16(raw[n]) for n in raw}

    last = {}

    def run(rows):
        t0 = time.perf_counter()
        last["res"] = nsa_ref.prefill(lz["q"], lz["k"], lz["v"], lz["gates"], block=cfg.block, top_k=cfg.top_k,
                                      window=cfg.window, rows=rows)
        return time.perf_counter() - t0

    L = cfg.seqlen
    # per-row cost from two probes (the difference removes the fixed per-call cost)
    t_small = run(np.linspace(0, L - 1, 8).astype(np.int64))
    t_big = run(np.linspace(0, L - 1, 72).astype(np.int64))
    per_row = max((t_big - t_small) / 64, 1e-5)
    fixed = max(t_small - 8 * per_row, 0.0)
    n_rows = int(max(16, min(20000, (seconds - fixed) / per_row)))
    rows = np.linspace(0, L - 1, n_rows).astype(np.int64)
    dt = run(rows)
    parity = None
    if gpu is not None:
        res = last["res"]
        g_out, g_idx = gpu
        import torch
        rsel = torch.as_tensor(rows, device=g_out.device)
        go = g_out[:, rsel].float().cpu().numpy().astype(np.float64)
        gi = g_idx[:, rsel].cpu().numpy()
        expect = res["out"].copy()
        differ = np.argwhere(np.any(gi != res["idx"], axis=(2, 3)))
        for b, r in differ:
            inj = np.zeros((1, L, cfg.n_kv_heads, cfg.top_k), np.int32)
            inj[0, rows[r]] = gi[b, r]
            lb = {n: _LazyBf16(raw[n][b:b + 1]) for n in ("q", "k", "v", "gates")}
            expect[b, r] = nsa_ref.prefill(lb["q"], lb["k"], lb["v"], lb["gates"], block=cfg.block,
                                           top_k=cfg.top_k, window=cfg.window, rows=[rows[r]],
                                           inject_idx=inj)["out"][0, 0]
        parity = {"rows": int(n_rows * cfg.batch), "rows_with_the_oracle_selection": int(n_rows * cfg.batch - len(differ)),
                  "out_dtype": "bf16", "max_abs_err": float(np.max(np.abs(go - expect))), "tol": 2e-2,
                  "note": "rows whose selection differs are compared with the oracle given the library's selection"}
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    return {"value": n_rows * cfg.batch / dt, "unit": "tokens/s", "cores": ncores, "kind": "oracle",
            "cpu_model": cpu_model, "blas": blas,
            "sample": f"{n_rows} evenly spaced query rows of the {cfg.name} workload (full "
                      f"{L}-token context, all {cfg.n_q_heads} heads), float64 numpy, {dt:.1f} s",
            "parity_of_timed_output": parity}


# ---------------------------------------------------------------- benchmark legs

def bench_prefill(cfg, steps, warmup, torch, inputs, nsa, raw=None):
    dev = torch.device("cuda:0")
    if raw is None:
        t0 = time.perf_counter()
        raw = inputs.make_prefill_inputs(cfg)
        log(f"[bench] inputs {cfg.name} generated in {time.perf_counter() - t0:.1f} s")
    up = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v, g = (up(raw[n]) for n in ("q", "k", "v", "gates"))
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    nbytes = nsa.prefill_workspace_bytes(q, k, v, g, out, top_k=cfg.top_k, window=cfg.window)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    call = lambda: nsa.prefill(q, k, v, g, top_k=cfg.top_k, window=cfg.window, out=out, workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    log(f"[bench] prefill {cfg.name}: {wall_ms:.3f} ms/step over {steps} steps")

    # per-kernel durations: the timed entry point records HIP events on the stream
    ns = len(PREFILL_STAGES) + 1
    ev = HipEvents(ns * steps)
    desc = nsa.prefill_desc(q, k, v, g, out)
    params = nsa.make_params(cfg.top_k, cfg.window)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    for i in range(steps):
        nsa.check(nsa.lib().nsa_fwd_prefill_timed(
            ctypes.byref(desc), ctypes.byref(params), ctypes.c_void_p(q.data_ptr()),
            ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(g.data_ptr()),
            ctypes.c_void_p(out.data_ptr()), None, nsa.NSA_IDX_COMPUTE, ctypes.c_void_p(ws.data_ptr()),
            ws.numel(), stream, ev.array(i * ns, ns)))
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([ev.elapsed_ms(i * ns + s, i * ns + s + 1) for i in range(steps)]))
                for s, name in enumerate(PREFILL_STAGES)}
    ev.close()
    return raw, wall_ms, stage_ms


def bench_chunked(cfg, raw, chunk, steps, warmup, torch, nsa):
    """The same prefill as a sequence of nsa_fwd_prefill_chunk calls over
    query chunks of `chunk` positions, each against the context up to its
    end (one step = all chunks); outputs land in one [B, L, Hq, D] tensor."""
    dev = torch.device("cuda:0")
    up = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v, g = (up(raw[n]) for n in ("q", "k", "v", "gates"))
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(nsa.prefill_workspace_bytes(q, k, v, g, out, top_k=cfg.top_k, window=cfg.window),
                     dtype=torch.uint8, device=dev)
    L = cfg.seqlen
    bounds = list(range(0, L, chunk)) + [L]

    def step():
        for t0, t1 in zip(bounds[:-1], bounds[1:]):
            nsa.prefill_chunk(q[:, t0:t1], k[:, :t1], v[:, :t1], g[:, t0:t1], t0, top_k=cfg.top_k,
                              window=cfg.window, out=out[:, t0:t1], workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    log(f"[bench] chunked prefill {cfg.name} in chunks of {chunk}: {ms:.3f} ms per pass")
    return {"chunk": chunk, "calls": len(bounds) - 1, "ms_per_pass": ms,
            "tokens_per_s": cfg.batch * L / (ms * 1e-3)}


def bench_varlen(cfg, raw, steps, warmup, torch, nsa):
    """One nsa_fwd_prefill_varlen call over four sequences of 1, 3/4, 1/2 and
    1/4 of the main config's length (all views of its inputs, batch stride 0);
    each sequence's queries are its whole length."""
    dev = torch.device("cuda:0")
    up = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v, g = (up(raw[n]) for n in ("q", "k", "v", "gates"))
    L = cfg.seqlen
    lens = [L, 3 * L // 4, L // 2, L // 4]
    nb = len(lens)
    q4, k4, v4, g4 = (t.expand(nb, *t.shape[1:]) for t in (q, k, v, g))
    out = torch.empty((nb,) + tuple(q.shape[1:]), dtype=torch.bfloat16, device=dev)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    ws = torch.empty(nsa.prefill_workspace_bytes(q4, k4, v4, g4, out, top_k=cfg.top_k, window=cfg.window),
                     dtype=torch.uint8, device=dev)
    call = lambda: nsa.prefill_varlen(q4, k4, v4, g4, sl, None, top_k=cfg.top_k, window=cfg.window, out=out,
                                      workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    log(f"[bench] varlen prefill {lens}: {ms:.3f} ms per call")
    return {"seq_lens": lens, "ms_per_call": ms, "tokens_per_s": sum(lens) / (ms * 1e-3)}


def bench_shared_selection(cfg, raw, steps, torch, nsa):
    """The main config with an injected selection in which the 64 query
    tokens of each block share one random set of earlier blocks per KV group
    (plus their own block): a stand-in for the locality of real text, where
    neighbouring tokens read the same passages. A separate, clearly labelled
    run; per-kernel times as in the main run."""
    dev = torch.device("cuda:0")
    up = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v, g = (up(raw[n]) for n in ("q", "k", "v", "gates"))
    B, L, G, n = cfg.batch, cfg.seqlen, cfg.n_kv_heads, cfg.top_k
    rng = np.random.default_rng(1)
    nqb = (L + 63) // 64
    rows = np.full((B, nqb, G, n), -1, dtype=np.int32)
    for b in range(B):
        for qb in range(nqb):
            m = min(n - 1, qb)
            for gg in range(G):
                rows[b, qb, gg, :m + 1] = np.sort(np.append(rng.choice(qb, m, replace=False), qb))
    idx = torch.from_numpy(np.ascontiguousarray(np.repeat(rows, 64, axis=1)[:, :L])).to(dev)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(nsa.prefill_workspace_bytes(q, k, v, g, out, top_k=n, window=cfg.window), dtype=torch.uint8,
                     device=dev)
    ns = len(PREFILL_STAGES) + 1
    ev = HipEvents(ns * steps)
    desc = nsa.prefill_desc(q, k, v, g, out)
    params = nsa.make_params(n, cfg.window)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    call = lambda evs: nsa.check(nsa.lib().nsa_fwd_prefill_timed(
        ctypes.byref(desc), ctypes.byref(params), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
        ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(g.data_ptr()), ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(idx.data_ptr()), nsa.NSA_IDX_INJECT, ctypes.c_void_p(ws.data_ptr()), ws.numel(), stream,
        evs))
    call(ev.array(0, ns))  # warm-up
    torch.cuda.synchronize()
    for i in range(steps):
        call(ev.array(i * ns, ns))
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([ev.elapsed_ms(i * ns + s_, i * ns + s_ + 1) for i in range(steps)]))
                for s_, name in enumerate(PREFILL_STAGES)}
    ev.close()
    log(f"[bench] shared-selection prefill {cfg.name}: kernels {stage_ms}")
    return {"selection": "injected; the 64 query tokens of a block share one random block set per KV group",
            "kernels_ms": stage_ms, "note": "not the headline workload (its selection is computed)"}


def bench_backward(cfg, raw, steps, torch, nsa):
    """nsa_bwd_prefill on the main config: the selection is the forward's own
    (computed by nsa_fwd_prefill on the same inputs), dout a seeded bf16
    normal draw made on the GPU. Algorithmic work: the five products of
    attention's backward (S, dP, dq, dK, dV) over every (query, key, head)
    the forward visits, 2.5 times the forward's flops; the query-side kernel
    also recomputes each branch's forward (S and P.V once more)."""
    dev = torch.device("cuda:0")
    up = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v, g = (up(raw[n]) for n in ("q", "k", "v", "gates"))
    B, L, Hq, D = q.shape
    G = k.shape[2]
    out, idx = nsa.prefill(q, k, v, g, top_k=cfg.top_k, window=cfg.window, return_idx=True)
    del out
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    dout = torch.randn(q.shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    f32 = dict(dtype=torch.float32, device=dev)
    grads = (torch.empty((B, L, Hq, D), **f32), torch.empty((B, L, G, D), **f32),
             torch.empty((B, L, G, D), **f32), torch.empty((B, L, Hq, 3), **f32))
    ws = torch.empty(nsa.prefill_backward_workspace_bytes(q, k, v, g, dout, top_k=cfg.top_k, window=cfg.window),
                     dtype=torch.uint8, device=dev)
    desc = nsa.prefill_desc(q, k, v, g, dout)
    params = nsa.make_params(cfg.top_k, cfg.window)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    ns = len(BACKWARD_STAGES) + 1
    ev = HipEvents(ns * steps)
    call = lambda evs: nsa.check(nsa.lib().nsa_bwd_prefill_timed(
        ctypes.byref(desc), ctypes.byref(params), P(q), P(k), P(v), P(g), P(dout), P(idx), *(P(x) for x in grads),
        P(ws), ws.numel(), stream, evs))
    call(ev.array(0, ns))  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        call(ev.array(i * ns, ns))
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    stage_ms = {name: float(np.mean([ev.elapsed_ms(i * ns + s_, i * ns + s_ + 1) for i in range(steps)]))
                for s_, name in enumerate(BACKWARD_STAGES)}
    ev.close()
    fl = 2.5 * sum(prefill_flops(cfg).values())
    log(f"[bench] backward {cfg.name}: {wall_ms:.3f} ms/step over {steps} steps, kernels {stage_ms}")

    # the training path: nsa_fwd_prefill_save keeps the selected branch's
    # output and log-sum-exp, and nsa_bwd_prefill_saved uses them
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        _, idx_s, saved = nsa.prefill_save(q, k, v, g, top_k=cfg.top_k, window=cfg.window)
    torch.cuda.synchronize()
    save_ms = (time.perf_counter() - t0) * 1e3 / steps
    o_slc, lse_slc = saved
    ev = HipEvents(ns * steps)
    call_s = lambda evs: nsa.check(nsa.lib().nsa_bwd_prefill_saved_timed(
        ctypes.byref(desc), ctypes.byref(params), P(q), P(k), P(v), P(g), P(dout), P(idx_s), P(o_slc), P(lse_slc),
        *(P(x) for x in grads), P(ws), ws.numel(), stream, evs))
    call_s(ev.array(0, ns))  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        call_s(ev.array(i * ns, ns))
    torch.cuda.synchronize()
    saved_ms = (time.perf_counter() - t0) * 1e3 / steps
    saved_stage = {name: float(np.mean([ev.elapsed_ms(i * ns + s_, i * ns + s_ + 1) for i in range(steps)]))
                   for s_, name in enumerate(BACKWARD_STAGES)}
    ev.close()
    log(f"[bench] backward {cfg.name} from the saved selected branch: {saved_ms:.3f} ms/step, kernels "
        f"{saved_stage}; the saving forward {save_ms:.3f} ms/step")
    return {"workload": f"nsa_prefill_backward_{cfg.name}", "ms_per_step": wall_ms,
            "tokens_per_s": cfg.batch * cfg.seqlen / (wall_ms * 1e-3), "kernels_ms": stage_ms,
            "algorithmic_flops": fl, "tflops": fl / (wall_ms * 1e-3) / 1e12,
            "mfma_frac": fl / (wall_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "selection": "the forward's computed selection", "dout": "seeded bf16 normal draw",
            "outputs": "fp32 dq, dk, dv, dgates",
            "saved": {"entry": "nsa_bwd_prefill_saved after nsa_fwd_prefill_save", "ms_per_step": saved_ms,
                      "kernels_ms": saved_stage, "tflops": fl / (saved_ms * 1e-3) / 1e12,
                      "mfma_frac": fl / (saved_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                      "forward_save_ms_per_step": save_ms}}


def dsa_flops(cfg):
    """Algorithmic work of token-level sparse attention: the indexer's dot
    products (2 Di per (query, earlier token, indexer head)) and the attention
    over the chosen tokens (4 D per (query, chosen token, query head))."""
    L, k = cfg.seqlen, cfg.top_k
    t = np.arange(L, dtype=np.int64)
    pairs = int((t + 1).sum())
    chosen = int(np.minimum(t + 1, k).sum())
    return {"indexer": cfg.batch * pairs * cfg.idx_heads * 2 * cfg.idx_dim,
            "attention": cfg.batch * chosen * cfg.n_q_heads * 4 * cfg.head_dim,
            "score_bytes": cfg.batch * pairs * 4, "chosen": cfg.batch * chosen}


def bench_dsa(cfg, steps, warmup, torch, inputs, nsa):
    """nsa_dsa_prefill (indexer, top-k, attention over the chosen tokens) on
    the token-level sparse workload, timed per stage with HIP events."""
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    raw = inputs.make_dsa_inputs(cfg)
    log(f"[bench] inputs {cfg.name} generated in {time.perf_counter() - t0:.1f} s")
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    ts = [up(raw[n]) for n in ("q", "k", "v", "qi", "ki", "w")]
    del raw
    out = torch.empty(ts[0].shape, dtype=torch.bfloat16, device=dev)
    idx = torch.empty((cfg.batch, cfg.seqlen, cfg.top_k), dtype=torch.int32, device=dev)
    ws = torch.empty(nsa.dsa_workspace_bytes(*ts, out, top_k=cfg.top_k), dtype=torch.uint8, device=dev)
    desc = nsa.dsa_desc(*ts, out)
    params = nsa.DsaParams(cfg.top_k, 0.0)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    call = lambda: nsa.dsa_prefill(*ts, top_k=cfg.top_k, out=out, idx=idx, workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    stages = ["indexer", "topk", "attention"]
    ns = len(stages) + 1
    ev = HipEvents(ns * steps)
    for i in range(steps):
        nsa.check(nsa.lib().nsa_dsa_prefill_timed(ctypes.byref(desc), ctypes.byref(params), *(P(x) for x in ts), P(out),
                                                  P(idx), nsa.NSA_IDX_COMPUTE, P(ws), ws.numel(), stream,
                                                  ev.array(i * ns, ns)))
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([ev.elapsed_ms(i * ns + s, i * ns + s + 1) for i in range(steps)]))
                for s, name in enumerate(stages)}
    ev.close()
    fl = dsa_flops(cfg)
    gathered = fl["chosen"] * cfg.n_kv_heads * cfg.head_dim * 2 * 2
    log(f"[bench] dsa {cfg.name}: {wall_ms:.3f} ms/step, kernels {stage_ms}")
    return {"workload": cfg.name, "batch": cfg.batch, "seqlen": cfg.seqlen, "top_k": cfg.top_k,
            "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
            "idx_heads": cfg.idx_heads, "idx_dim": cfg.idx_dim, "ms_per_step": wall_ms,
            "tokens_per_s": cfg.batch * cfg.seqlen / (wall_ms * 1e-3), "kernels_ms": stage_ms,
            "indexer": {"flops": fl["indexer"], "tflops": fl["indexer"] / (stage_ms["indexer"] * 1e-3) / 1e12,
                        "mfma_frac": fl["indexer"] / (stage_ms["indexer"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                        "score_bytes_written": fl["score_bytes"]},
            "topk": {"score_bytes_read": fl["score_bytes"],
                     "GBps": fl["score_bytes"] / (stage_ms["topk"] * 1e-3) / 1e9},
            "attention": {"flops": fl["attention"],
                          "tflops": fl["attention"] / (stage_ms["attention"] * 1e-3) / 1e12,
                          "mfma_frac": fl["attention"] / (stage_ms["attention"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                          "gathered_bytes": gathered,
                          "gathered_TBps": gathered / (stage_ms["attention"] * 1e-3) / 1e12},
            "dtype": "bf16 (indexer and attention operands), fp32 scores and accumulation",
            "traffic": {kn: committed_traffic(kn, cfg.name, "dsa")
                        for kn in ("k_dsa_index", "k_dsa_topk_fast", "k_dsa_topk_exact", "k_dsa_attn")}}


def bench_decode(cfg, steps, warmup, torch, inputs, nsa, general=False):
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    raw = inputs.make_decode_inputs(cfg)
    log(f"[bench] inputs {cfg.name} generated in {time.perf_counter() - t0:.1f} s")
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    q, g = up(raw["q"]), up(raw["gates"])
    kc = up(raw["k_cache"])
    vc = up(raw["v_cache"])
    del raw["k_cache"], raw["v_cache"]
    lens = torch.from_numpy(raw["seqlens"]).to(dev)
    kb, vb = nsa.compress_kv(kc, vc)        # the block-mean cache, built by the library
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    idx = torch.empty((cfg.batch, cfg.n_kv_heads, cfg.top_k), dtype=torch.int32, device=dev)
    # read (not write) 1 GiB between steps: evicts the 256 MB Infinity Cache
    # without leaving dirty lines to be written back during the timed step
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    call = lambda: nsa.decode(q, kc, vc, kb, vb, lens, g, top_k=cfg.top_k, window=cfg.window, out=out,
                              idx=idx)
    for _ in range(warmup):
        call()
    ns = len(DECODE_STAGES) + 1
    ev = HipEvents(ns * steps)
    desc = nsa.decode_desc(q, kc, vc, kb, vb, g, out)
    params = nsa.make_params(cfg.top_k, cfg.window)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    nbytes = ctypes.c_size_t()
    nsa.check(nsa.lib().nsa_decode_workspace_bytes(ctypes.byref(desc), ctypes.byref(params), ctypes.byref(nbytes)))
    ws = torch.empty(nbytes.value, dtype=torch.uint8, device=dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    for i in range(steps):
        flush_sum = flush.sum()                # evict the previous step's data from the caches
        nsa.check(nsa.lib().nsa_fwd_decode_timed(
            ctypes.byref(desc), ctypes.byref(params), P(q), P(kc), P(vc), P(kb), P(vb), P(lens), P(g),
            P(out), P(idx), nsa.NSA_IDX_COMPUTE, P(ws), ws.numel(), stream, ev.array(i * ns, ns)))
    torch.cuda.synchronize()
    step_ms = [ev.elapsed_ms(i * ns, i * ns + ns - 1) for i in range(steps)]
    stage_ms = {name: float(np.mean([ev.elapsed_ms(i * ns + s, i * ns + s + 1) for i in range(steps)]))
                for s, name in enumerate(DECODE_STAGES)}
    ev.close()
    ubytes = decode_unique_bytes(cfg, idx.cpu().numpy(), raw["seqlens"])
    ms = float(np.median(step_ms))
    gbps = ubytes / (ms * 1e-3) / 1e9
    log(f"[bench] decode {cfg.name}: {ms * 1e3:.1f} us/step, {gbps:.0f} GB/s")
    res = {"workload": cfg.name, "ms_per_step": ms, "step_ms_samples": step_ms,
           "sequences_per_s": cfg.batch / (ms * 1e-3), "unique_bytes_per_step": ubytes,
           "achieved_GBps": gbps, "hbm_frac": gbps / PEAK_HBM_GBPS, "kernels_ms": stage_ms,
           "traffic": committed_traffic("k_dec", cfg.name), "cache_flush": "1 GiB read between steps"}
    if general:
        res["general"] = bench_decode_general(cfg, q, kc, vc, lens, g, flush, raw["seqlens"], steps, torch, nsa)
    return res


GENERAL = {"block": 32, "stride": 16, "select_block": 64}   # the overlapping geometry the general legs time


def bench_decode_general(cfg, q, kc, vc, lens, g, flush, seqlens, steps, torch, nsa):
    """The decode with the general geometry (nsa_fwd_decode_general) on the
    same caches: blocks of 32 tokens at stride 16 (their means built once with
    torch, outside the timing), selection blocks of 64; HIP events around
    each call after the 1 GiB flush."""
    l, d, ls = GENERAL["block"], GENERAL["stride"], GENERAL["select_block"]

    def block_means(c):   # blocks of 2d tokens at stride d: the average of two neighbouring d-token means
        B, G, L, D = c.shape
        m = c.view(B, G, L // d, d, D).float().mean(3)
        return ((m[:, :, :-1] + m[:, :, 1:]) * 0.5).to(torch.bfloat16).contiguous()

    assert l == 2 * d and cfg.max_seqlen % d == 0
    kb, vb = block_means(kc), block_means(vc)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    idx = torch.empty((cfg.batch, cfg.n_kv_heads, cfg.top_k), dtype=torch.int32, device=q.device)
    call = lambda: nsa.decode_general(q, kc, vc, kb, vb, lens, g, top_k=cfg.top_k, window=cfg.window, block=l,
                                      select_block=ls, stride=d, out=out, idx=idx)
    for _ in range(3):
        call()
    times = []
    for _ in range(steps):
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    ubytes = decode_unique_bytes(cfg, idx.cpu().numpy(), seqlens, cl=l, cd=d, ls=ls)
    gbps = ubytes / (ms * 1e-3) / 1e9
    log(f"[bench] decode {cfg.name}, general geometry {GENERAL}: {ms * 1e3:.1f} us/step, {gbps:.0f} GB/s")
    return {"entry": "nsa_fwd_decode_general", "geometry": dict(GENERAL), "ms_per_step": ms,
            "unique_bytes_per_step": ubytes, "achieved_GBps": gbps, "hbm_frac": gbps / PEAK_HBM_GBPS,
            "timing": "HIP events around each call (launch included), 1 GiB read between calls"}


def bench_prefill_general(cfg, raw, steps, torch, nsa):
    """The prefill with the general geometry (nsa_fwd_prefill_general) on the
    main config's inputs: blocks of 32 tokens at stride 16 (twice the
    compressed blocks, overlapping), selection blocks of 64, block means."""
    dev = torch.device("cuda:0")
    l, d, ls = GENERAL["block"], GENERAL["stride"], GENERAL["select_block"]
    up = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v, g = (up(raw[n]) for n in ("q", "k", "v", "gates"))
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    call = lambda: nsa.prefill_general(q, k, v, g, top_k=cfg.top_k, window=cfg.window, block=l, select_block=ls,
                                       stride=d, out=out)
    call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    log(f"[bench] prefill {cfg.name}, general geometry {GENERAL}: {ms:.3f} ms/step")
    return {"entry": "nsa_fwd_prefill_general", "geometry": dict(GENERAL), "ms_per_step": ms,
            "tokens_per_s": cfg.batch * cfg.seqlen / (ms * 1e-3)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="p64k", choices=["p8k", "p32k", "p64k"])
    ap.add_argument("--chunk", type=int, default=8192,
                    help="also time the main config as chunked prefill calls of this many query "
                         "positions (0: skip)")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the varlen prefill of four sequences of mixed lengths")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward pass of the main config")
    ap.add_argument("--no-shared-selection", action="store_true",
                    help="skip the run with an injected selection shared by neighbouring tokens")
    ap.add_argument("--also", default="p8k,p32k",
                    help="shorter prefill configs also reported (their inputs are prefixes of the "
                         "main config's); empty for none")
    ap.add_argument("--dsa", default="dsa64k", help="token-level sparse attention workload also timed ('' to skip)")
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-general", action="store_true",
                    help="skip the prefill and decode with the general geometry (blocks of 32 at stride 16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run 3 plain fp32 copies of MIB MiB (a known HBM read + write "
                         "volume for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the NSA path here is single-GPU; sharding is described in the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from long_context_sparse_fwd_amd import inputs, nsa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    nsa.lib()
    if args.copy_calibration > 0:
        n = args.copy_calibration << 18  # fp32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 x (read {n * 4} B, write {n * 4} B)")
        del src, dst
    cfg = inputs.CONFIGS[args.config]
    raw, wall_ms, stage_ms = bench_prefill(cfg, args.steps, args.warmup, torch, inputs, nsa)
    fl = prefill_flops(cfg)
    total_fl = sum(fl.values())
    tokens_per_s = cfg.batch * cfg.seqlen / (wall_ms * 1e-3)

    kernel_flops = {"k_cmpwin": fl["cmp"] + fl["win"], "k_sel": fl["slc"]}
    dominant = max(stage_ms, key=stage_ms.get)
    if dominant in kernel_flops:
        achieved = kernel_flops[dominant] / (stage_ms[dominant] * 1e-3) / 1e12
        roof = {"kernel": dominant, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": committed_traffic(dominant, cfg.name),
                "work_per_launch": kernel_flops[dominant], "avg_launch_ms": stage_ms[dominant]}
    else:
        prep_bytes = 4 * cfg.batch * cfg.seqlen * cfg.n_kv_heads * cfg.head_dim * 2
        achieved = prep_bytes / (stage_ms[dominant] * 1e-3) / 1e9
        roof = {"kernel": dominant, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                "traffic": committed_traffic(dominant, cfg.name),
                "work_per_launch": prep_bytes, "avg_launch_ms": stage_ms[dominant]}

    # the selected branch is bound by gathering K/V, not by its MFMA work: its
    # gathered bytes (D bf16 of K and of V per selected (query token, KV group,
    # key)), their rate, the rate of its L2 misses (committed counters), and the
    # gather probe's ceiling for the same pattern
    slc_keys = pair_counts(cfg.seqlen, cfg.block, cfg.top_k, cfg.window)[1] * cfg.batch * cfg.n_kv_heads
    gathered = slc_keys * cfg.head_dim * 2 * 2
    sel_s = stage_ms["k_sel"] * 1e-3
    sel_traffic = committed_traffic("k_sel", cfg.name)
    gather = {"kernel": "k_sel", "gathered_bytes_per_launch": gathered,
              "gathered_TBps": gathered / sel_s / 1e12,
              "l2_miss_TBps": sel_traffic / sel_s / 1e12 if sel_traffic else None,
              "probe_random_gather_32MiB_TBps": probe_gather_ceiling()}

    result = {
        "metric": "NSA fwd prefill tokens/s & MFMA % peak at 64k; decode HBM GB/s % peak",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v, sigmoid(N(0,1)) gates)",
        "config": {"workload": f"nsa_prefill_{cfg.name}", "batch": cfg.batch, "seqlen": cfg.seqlen,
                   "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
                   "compress_block_size": cfg.block, "select_block_size": cfg.block,
                   "select_top_k": cfg.top_k, "sliding_window": cfg.window},
        "roofline": roof,
        "gather": gather,
        "prefill": {"tflops": total_fl / (wall_ms * 1e-3) / 1e12,
                    "mfma_frac": total_fl / (wall_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                    "algorithmic_flops": fl, "kernels_ms": stage_ms},
    }
    others = {}
    for name in [x for x in args.also.split(",") if x]:
        oc = inputs.CONFIGS[name]
        if oc.seqlen >= cfg.seqlen or oc.batch != cfg.batch:
            continue
        # the keyed generator makes the shorter config's inputs a prefix of these
        sub = {n: np.ascontiguousarray(raw[n][:, :oc.seqlen]) for n in ("q", "k", "v", "gates")}
        _, o_ms, o_stage = bench_prefill(oc, args.steps, args.warmup, torch, inputs, nsa, raw=sub)
        o_fl = sum(prefill_flops(oc).values())
        others[name] = {"ms_per_step": o_ms, "tokens_per_s": oc.batch * oc.seqlen / (o_ms * 1e-3),
                        "tflops": o_fl / (o_ms * 1e-3) / 1e12,
                        "mfma_frac": o_fl / (o_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "kernels_ms": o_stage}
    if others:
        result["other_prefill"] = others
    if args.chunk > 0:
        result["chunked_prefill"] = bench_chunked(cfg, raw, args.chunk, args.steps, args.warmup, torch, nsa)
    if not args.no_varlen:
        result["varlen_prefill"] = bench_varlen(cfg, raw, args.steps, args.warmup, torch, nsa)
    if not args.no_shared_selection:
        result["shared_selection_prefill"] = bench_shared_selection(cfg, raw, args.steps, torch, nsa)
    if not args.no_backward:
        result["backward"] = bench_backward(cfg, raw, max(1, min(args.steps, 5)), torch, nsa)
    if args.dsa:
        result["dsa"] = bench_dsa(inputs.DSA_CONFIGS[args.dsa], max(1, min(args.steps, 5)), 1, torch, inputs, nsa)
    if not args.no_general:
        result["general_prefill"] = bench_prefill_general(cfg, raw, max(1, min(args.steps, 5)), torch, nsa)
    if not args.no_decode:
        result["decode"] = bench_decode(inputs.CONFIGS["d64k"], args.decode_steps, 3, torch, inputs, nsa,
                                        general=not args.no_general)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        up = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        q, k, v, g = (up(raw[n]) for n in ("q", "k", "v", "gates"))
        gpu = nsa.prefill(q, k, v, g, top_k=cfg.top_k, window=cfg.window, out_dtype=torch.bfloat16, return_idx=True)
        torch.cuda.synchronize()
        del q, k, v, g
        result["cpu_baseline"] = cpu_baseline(cfg, raw, args.cpu_seconds, gpu=gpu)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
