"""Thin ctypes binding of libnsa (include/nsa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libnsa.so. PyTorch supplies device memory and the current stream.
There is no CPU fallback: calling into the library without the built .so or
without a GPU raises.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnsa.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "nsa.h")

NSA_OK, NSA_ERR_INVALID_ARGUMENT, NSA_ERR_UNSUPPORTED, NSA_ERR_WORKSPACE_TOO_SMALL, NSA_ERR_HIP = range(5)
NSA_F32, NSA_BF16 = 0, 1
NSA_IDX_COMPUTE, NSA_IDX_INJECT = 0, 1

c_i32, c_i64, c_f32, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class NsaParams(ctypes.Structure):
    _fields_ = [("compress_block_size", c_i32), ("select_block_size", c_i32),
                ("select_top_k", c_i32), ("sliding_window", c_i32), ("softmax_scale", c_f32)]


class PrefillDesc(ctypes.Structure):
    _fields_ = [("batch", c_i32), ("seqlen", c_i32), ("n_q_heads", c_i32), ("n_kv_heads", c_i32),
                ("head_dim", c_i32), ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("q_stride", c_i64 * 3), ("k_stride", c_i64 * 3), ("v_stride", c_i64 * 3),
                ("g_stride", c_i64 * 3), ("o_stride", c_i64 * 3)]


class DecodeDesc(ctypes.Structure):
    _fields_ = [("batch", c_i32), ("max_seqlen", c_i32), ("max_blocks", c_i32),
                ("n_q_heads", c_i32), ("n_kv_heads", c_i32), ("head_dim", c_i32),
                ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("q_stride", c_i64 * 2), ("k_stride", c_i64 * 3), ("v_stride", c_i64 * 3),
                ("kc_stride", c_i64 * 3), ("vc_stride", c_i64 * 3), ("g_stride", c_i64 * 2),
                ("o_stride", c_i64 * 2)]


class NsaGeneral(ctypes.Structure):
    _fields_ = [("compress_stride", c_i32), ("wk", c_vp), ("bk", c_vp), ("wv", c_vp), ("bv", c_vp),
                ("gate_w", c_vp), ("gate_b", c_vp)]


class DsaDesc(ctypes.Structure):
    _fields_ = [("batch", c_i32), ("seqlen", c_i32), ("n_q_heads", c_i32), ("n_kv_heads", c_i32),
                ("head_dim", c_i32), ("idx_heads", c_i32), ("idx_dim", c_i32), ("in_dtype", ctypes.c_int),
                ("out_dtype", ctypes.c_int), ("q_stride", c_i64 * 3), ("k_stride", c_i64 * 3),
                ("v_stride", c_i64 * 3), ("o_stride", c_i64 * 3), ("qi_stride", c_i64 * 3),
                ("ki_stride", c_i64 * 2), ("w_stride", c_i64 * 2)]


class DsaParams(ctypes.Structure):
    _fields_ = [("top_k", c_i32), ("softmax_scale", c_f32)]


class NsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libnsa.so (built in-tree by long_context_sparse_fwd_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m long_context_sparse_fwd_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.nsa_status_string.restype = ctypes.c_char_p
    L.nsa_status_string.argtypes = [ctypes.c_int]
    L.nsa_last_error.restype = ctypes.c_char_p
    L.nsa_last_error.argtypes = []
    L.nsa_version.restype = c_i32
    L.nsa_prefill_workspace_bytes.restype = ctypes.c_int
    L.nsa_prefill_workspace_bytes.argtypes = [P(PrefillDesc), P(NsaParams), P(ctypes.c_size_t)]
    L.nsa_decode_workspace_bytes.restype = ctypes.c_int
    L.nsa_decode_workspace_bytes.argtypes = [P(DecodeDesc), P(NsaParams), P(ctypes.c_size_t)]
    L.nsa_fwd_prefill.restype = ctypes.c_int
    L.nsa_fwd_prefill.argtypes = [P(PrefillDesc), P(NsaParams), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                  ctypes.c_int, c_vp, ctypes.c_size_t, c_vp]
    L.nsa_prefill_general_workspace_bytes.restype = ctypes.c_int
    L.nsa_prefill_general_workspace_bytes.argtypes = [P(PrefillDesc), P(NsaParams), P(NsaGeneral),
                                                      P(ctypes.c_size_t)]
    L.nsa_fwd_prefill_general.restype = ctypes.c_int
    L.nsa_fwd_prefill_general.argtypes = [P(PrefillDesc), P(NsaParams), P(NsaGeneral), c_vp, c_vp, c_vp, c_vp,
                                          c_vp, c_vp, ctypes.c_int, c_vp, ctypes.c_size_t, c_vp]
    L.nsa_fwd_prefill_chunk.restype = ctypes.c_int
    L.nsa_fwd_prefill_chunk.argtypes = [P(PrefillDesc), P(NsaParams), c_i32, c_vp, c_vp, c_vp, c_vp, c_vp,
                                        c_vp, ctypes.c_int, c_vp, ctypes.c_size_t, c_vp]
    L.nsa_fwd_prefill_varlen.restype = ctypes.c_int
    L.nsa_fwd_prefill_varlen.argtypes = [P(PrefillDesc), P(NsaParams), c_vp, c_vp, c_i32, c_vp, c_vp, c_vp,
                                         c_vp, c_vp, c_vp, ctypes.c_int, c_vp, ctypes.c_size_t, c_vp]
    L.nsa_fwd_decode.restype = ctypes.c_int
    L.nsa_fwd_decode.argtypes = [P(DecodeDesc), P(NsaParams), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                 c_vp, c_vp, c_vp, ctypes.c_int, c_vp, ctypes.c_size_t, c_vp]
    L.nsa_decode_general_workspace_bytes.restype = ctypes.c_int
    L.nsa_decode_general_workspace_bytes.argtypes = [P(DecodeDesc), P(NsaParams), P(NsaGeneral),
                                                     P(ctypes.c_size_t)]
    L.nsa_fwd_decode_general.restype = ctypes.c_int
    L.nsa_fwd_decode_general.argtypes = [P(DecodeDesc), P(NsaParams), P(NsaGeneral), c_vp, c_vp, c_vp, c_vp,
                                         c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_int, c_vp, ctypes.c_size_t, c_vp]
    L.nsa_fwd_decode_noalloc.restype = ctypes.c_int
    L.nsa_fwd_decode_noalloc.argtypes = [P(DecodeDesc), P(NsaParams), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                         c_vp, c_vp, c_vp, ctypes.c_int, c_vp]
    L.nsa_dsa_workspace_bytes.restype = ctypes.c_int
    L.nsa_dsa_workspace_bytes.argtypes = [P(DsaDesc), P(DsaParams), P(ctypes.c_size_t)]
    L.nsa_dsa_prefill.restype = ctypes.c_int
    L.nsa_dsa_prefill.argtypes = [P(DsaDesc), P(DsaParams), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                  ctypes.c_int, c_vp, ctypes.c_size_t, c_vp]
    L.nsa_dsa_prefill_timed.restype = ctypes.c_int
    L.nsa_dsa_prefill_timed.argtypes = L.nsa_dsa_prefill.argtypes + [c_vp]
    L.nsa_bwd_prefill_workspace_bytes.restype = ctypes.c_int
    L.nsa_bwd_prefill_workspace_bytes.argtypes = [P(PrefillDesc), P(NsaParams), P(ctypes.c_size_t)]
    L.nsa_bwd_prefill.restype = ctypes.c_int
    L.nsa_bwd_prefill.argtypes = [P(PrefillDesc), P(NsaParams), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                  c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]
    L.nsa_bwd_prefill_timed.restype = ctypes.c_int
    L.nsa_bwd_prefill_timed.argtypes = L.nsa_bwd_prefill.argtypes + [c_vp]
    L.nsa_bwd_prefill_saved.restype = ctypes.c_int
    L.nsa_bwd_prefill_saved.argtypes = [P(PrefillDesc), P(NsaParams), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                        c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]
    L.nsa_bwd_prefill_saved_timed.restype = ctypes.c_int
    L.nsa_bwd_prefill_saved_timed.argtypes = L.nsa_bwd_prefill_saved.argtypes + [c_vp]
    L.nsa_fwd_prefill_save.restype = ctypes.c_int
    L.nsa_fwd_prefill_save.argtypes = [P(PrefillDesc), P(NsaParams), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                       ctypes.c_int, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]
    L.nsa_compress_kv.restype = ctypes.c_int
    L.nsa_compress_kv.argtypes = [c_i32, c_i32, c_i32, c_i32, ctypes.c_int, c_i32, c_vp, P(c_i64),
                                  c_vp, P(c_i64), c_vp, P(c_i64), c_vp, P(c_i64), c_vp]
    _lib = L
    return L


def header_functions() -> list[str]:
    """Names of the functions include/nsa.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nsa_[a-z_0-9]+)\s*\(", text)))


def check(status: int) -> None:
    if status != NSA_OK:
        L = lib()
        raise NsaError(status, f"{L.nsa_status_string(status).decode()}: {L.nsa_last_error().decode()}")


def make_params(top_k: int, window: int, block: int = 64, select_block: int | None = None,
                scale: float = 0.0) -> NsaParams:
    return NsaParams(block, block if select_block is None else select_block, top_k, window, scale)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return NSA_BF16
    if dt == torch.float32:
        return NSA_F32
    raise TypeError(f"unsupported dtype {dt}")


def _stream_of(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require_gpu(*ts):
    for t in ts:
        if not t.is_cuda:
            raise RuntimeError("libnsa runs on the GPU only: pass device tensors")
        if t.stride(-1) != 1:
            raise ValueError("the last dimension must be contiguous")


def prefill_desc(q, k, v, gates, out) -> PrefillDesc:
    B, L, Hq, D = q.shape
    G = k.shape[2]
    d = PrefillDesc()
    d.batch, d.seqlen, d.n_q_heads, d.n_kv_heads, d.head_dim = B, L, Hq, G, D
    d.in_dtype, d.out_dtype = _dtype_code(q.dtype), _dtype_code(out.dtype)
    d.q_stride[:] = q.stride()[:3]
    d.k_stride[:] = k.stride()[:3]
    d.v_stride[:] = v.stride()[:3]
    d.g_stride[:] = gates.stride()[:3]
    d.o_stride[:] = out.stride()[:3]
    return d


def prefill(q, k, v, gates, *, top_k: int, window: int, block: int = 64, select_block=None,
            scale: float = 0.0, out=None, out_dtype=None, idx=None, inject: bool = False,
            return_idx: bool = False, workspace=None):
    """NSA prefill. q [B,L,Hq,D], k/v [B,L,G,D], gates [B,L,Hq,3] (device tensors).

    Returns out (and idx [B,L,G,top_k] int32 when return_idx or idx is given).
    With inject=True, idx supplies the block selection.
    """
    _require_gpu(q, k, v, gates)
    B, L, Hq, D = q.shape
    G = k.shape[2]
    if k.shape != (B, L, G, D) or v.shape != k.shape or gates.shape != (B, L, Hq, 3):
        raise ValueError("shape mismatch among q, k, v, gates")
    if not (q.dtype == k.dtype == v.dtype == gates.dtype):
        raise TypeError("q, k, v and gates must share one dtype")
    if out is None:
        out = torch.empty((B, L, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    if inject and idx is None:
        raise ValueError("inject=True needs idx")
    if idx is None and return_idx:
        idx = torch.empty((B, L, G, top_k), dtype=torch.int32, device=q.device)
    if idx is not None and (idx.dtype != torch.int32 or not idx.is_contiguous()
                            or tuple(idx.shape) != (B, L, G, top_k)):
        raise ValueError("idx must be a contiguous int32 [B, L, G, top_k] tensor")
    desc = prefill_desc(q, k, v, gates, out)
    params = make_params(top_k, window, block, select_block, scale)
    L_ = lib()
    nbytes = ctypes.c_size_t()
    check(L_.nsa_prefill_workspace_bytes(ctypes.byref(desc), ctypes.byref(params), ctypes.byref(nbytes)))
    if workspace is None or workspace.numel() < nbytes.value:
        workspace = torch.empty(max(nbytes.value, 1), dtype=torch.uint8, device=q.device)
    check(L_.nsa_fwd_prefill(ctypes.byref(desc), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v),
                             _ptr(gates), _ptr(out), _ptr(idx),
                             NSA_IDX_INJECT if inject else NSA_IDX_COMPUTE, _ptr(workspace),
                             workspace.numel(), _stream_of(q)))
    if idx is not None:
        return out, idx
    return out


def make_general(stride: int, compressor=None, gate_layer=None) -> NsaGeneral:
    """compressor: (wk, bk, wv, bv) device tensors or None; gate_layer:
    (gate_w, gate_b) or None. The tensors must outlive the call."""
    g = NsaGeneral()
    g.compress_stride = stride
    if compressor is not None:
        for name, t in zip(("wk", "bk", "wv", "bv"), compressor):
            if not (t.is_cuda and t.is_contiguous()):
                raise ValueError("compressor weights must be contiguous device tensors")
            setattr(g, name, t.data_ptr())
    if gate_layer is not None:
        for name, t in zip(("gate_w", "gate_b"), gate_layer):
            if not (t.is_cuda and t.is_contiguous()):
                raise ValueError("gate layer weights must be contiguous device tensors")
            setattr(g, name, t.data_ptr())
    return g


def prefill_general(q, k, v, gates, *, top_k: int, window: int, block: int = 64, select_block=None,
                    stride=None, compressor=None, gate_layer=None, scale: float = 0.0, out=None, out_dtype=None,
                    idx=None, inject: bool = False, return_idx: bool = False, workspace=None):
    """NSA prefill with the general geometry (nsa_fwd_prefill_general):
    compression stride, selection blocks of select_block tokens, a learned
    compressor (wk [D,block,D], bk [D], wv, bv) and a gate layer (gate_w
    [Hq,D,3], gate_b [Hq,3]); with a gate layer, gates may be None."""
    tensors = [q, k, v] + ([gates] if gates is not None else [])
    _require_gpu(*tensors)
    B, L, Hq, D = q.shape
    G = k.shape[2]
    if k.shape != (B, L, G, D) or v.shape != k.shape or (gates is not None and gates.shape != (B, L, Hq, 3)):
        raise ValueError("shape mismatch among q, k, v, gates")
    if gates is None and gate_layer is None:
        raise ValueError("gates are needed unless a gate layer computes them")
    for t in tensors + list(compressor or ()) + list(gate_layer or ()):
        if t.dtype != q.dtype:
            raise TypeError("inputs and weights must share one dtype")
    if out is None:
        out = torch.empty((B, L, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    if inject and idx is None:
        raise ValueError("inject=True needs idx")
    if idx is None and return_idx:
        idx = torch.empty((B, L, G, top_k), dtype=torch.int32, device=q.device)
    if idx is not None and (idx.dtype != torch.int32 or not idx.is_contiguous()
                            or tuple(idx.shape) != (B, L, G, top_k)):
        raise ValueError("idx must be a contiguous int32 [B, L, G, top_k] tensor")
    desc = prefill_desc(q, k, v, gates if gates is not None else q[..., :3], out)
    params = make_params(top_k, window, block, select_block, scale)
    gen = make_general(block if stride is None else stride, compressor, gate_layer)
    L_ = lib()
    nbytes = ctypes.c_size_t()
    check(L_.nsa_prefill_general_workspace_bytes(ctypes.byref(desc), ctypes.byref(params), ctypes.byref(gen),
                                                 ctypes.byref(nbytes)))
    if workspace is None or workspace.numel() < nbytes.value:
        workspace = torch.empty(max(nbytes.value, 1), dtype=torch.uint8, device=q.device)
    check(L_.nsa_fwd_prefill_general(ctypes.byref(desc), ctypes.byref(params), ctypes.byref(gen), _ptr(q), _ptr(k),
                                     _ptr(v), _ptr(gates), _ptr(out), _ptr(idx),
                                     NSA_IDX_INJECT if inject else NSA_IDX_COMPUTE, _ptr(workspace),
                                     workspace.numel(), _stream_of(q)))
    if idx is not None:
        return out, idx
    return out


def prefill_chunk(q, k, v, gates, q_offset: int, *, top_k: int, window: int, block: int = 64,
                  select_block=None, scale: float = 0.0, out=None, out_dtype=None, idx=None,
                  inject: bool = False, return_idx: bool = False, workspace=None):
    """Chunked NSA prefill: query positions [q_offset, L) against the L-token
    context. q [B,Lq,Hq,D] and gates [B,Lq,Hq,3] hold the Lq = L - q_offset
    query rows, k/v [B,L,G,D] the whole context; out (and idx [B,Lq,G,top_k])
    have the query rows."""
    _require_gpu(q, k, v, gates)
    B, Lq, Hq, D = q.shape
    _, L, G, _ = k.shape
    if L - q_offset != Lq or k.shape != (B, L, G, D) or v.shape != k.shape or gates.shape != (B, Lq, Hq, 3):
        raise ValueError("shape mismatch among q, k, v, gates and q_offset")
    if not (q.dtype == k.dtype == v.dtype == gates.dtype):
        raise TypeError("q, k, v and gates must share one dtype")
    if out is None:
        out = torch.empty((B, Lq, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    if inject and idx is None:
        raise ValueError("inject=True needs idx")
    if idx is None and return_idx:
        idx = torch.empty((B, Lq, G, top_k), dtype=torch.int32, device=q.device)
    if idx is not None and (idx.dtype != torch.int32 or not idx.is_contiguous()
                            or tuple(idx.shape) != (B, Lq, G, top_k)):
        raise ValueError("idx must be a contiguous int32 [B, Lq, G, top_k] tensor")
    desc = prefill_desc(q, k, v, gates, out)
    desc.seqlen = L
    params = make_params(top_k, window, block, select_block, scale)
    L_ = lib()
    nbytes = ctypes.c_size_t()
    check(L_.nsa_prefill_workspace_bytes(ctypes.byref(desc), ctypes.byref(params), ctypes.byref(nbytes)))
    if workspace is None or workspace.numel() < nbytes.value:
        workspace = torch.empty(max(nbytes.value, 1), dtype=torch.uint8, device=q.device)
    check(L_.nsa_fwd_prefill_chunk(ctypes.byref(desc), ctypes.byref(params), q_offset, _ptr(q), _ptr(k),
                                   _ptr(v), _ptr(gates), _ptr(out), _ptr(idx),
                                   NSA_IDX_INJECT if inject else NSA_IDX_COMPUTE, _ptr(workspace),
                                   workspace.numel(), _stream_of(q)))
    if idx is not None:
        return out, idx
    return out


def prefill_varlen(q, k, v, gates, seq_lens, q_offsets=None, *, top_k: int, window: int, block: int = 64,
                   select_block=None, scale: float = 0.0, out=None, out_dtype=None, idx=None,
                   inject: bool = False, return_idx: bool = False, workspace=None):
    """Varlen NSA prefill. k/v [B,L,G,D] hold up to L context rows per
    sequence; seq_lens [B] and q_offsets [B] (int32 device tensors) give each
    sequence's context length and first query position; q [B,R,Hq,D] and
    gates [B,R,Hq,3] hold R query rows per sequence (row i = position
    q_offsets[b] + i). out (and idx [B,R,G,top_k]) get those rows; rows past a
    sequence's queries are left as they are."""
    _require_gpu(q, k, v, gates, seq_lens)
    B, R, Hq, D = q.shape
    _, L, G, _ = k.shape
    if R > L or k.shape != (B, L, G, D) or v.shape != k.shape or gates.shape != (B, R, Hq, 3):
        raise ValueError("shape mismatch among q, k, v and gates")
    for t in (seq_lens,) + ((q_offsets,) if q_offsets is not None else ()):
        if t.dtype != torch.int32 or tuple(t.shape) != (B,) or not t.is_contiguous():
            raise ValueError("seq_lens / q_offsets must be contiguous int32 [B] tensors")
    if not (q.dtype == k.dtype == v.dtype == gates.dtype):
        raise TypeError("q, k, v and gates must share one dtype")
    if out is None:
        out = torch.zeros((B, R, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    if inject and idx is None:
        raise ValueError("inject=True needs idx")
    if idx is None and return_idx:
        idx = torch.full((B, R, G, top_k), -1, dtype=torch.int32, device=q.device)
    if idx is not None and (idx.dtype != torch.int32 or not idx.is_contiguous()
                            or tuple(idx.shape) != (B, R, G, top_k)):
        raise ValueError("idx must be a contiguous int32 [B, R, G, top_k] tensor")
    desc = prefill_desc(q, k, v, gates, out)
    desc.seqlen = L
    params = make_params(top_k, window, block, select_block, scale)
    L_ = lib()
    nbytes = ctypes.c_size_t()
    check(L_.nsa_prefill_workspace_bytes(ctypes.byref(desc), ctypes.byref(params), ctypes.byref(nbytes)))
    if workspace is None or workspace.numel() < nbytes.value:
        workspace = torch.empty(max(nbytes.value, 1), dtype=torch.uint8, device=q.device)
    check(L_.nsa_fwd_prefill_varlen(ctypes.byref(desc), ctypes.byref(params), _ptr(seq_lens), _ptr(q_offsets),
                                    R, _ptr(q), _ptr(k), _ptr(v), _ptr(gates), _ptr(out), _ptr(idx),
                                    NSA_IDX_INJECT if inject else NSA_IDX_COMPUTE, _ptr(workspace),
                                    workspace.numel(), _stream_of(q)))
    if idx is not None:
        return out, idx
    return out


def prefill_workspace_bytes(q, k, v, gates, out, *, top_k, window, block=64) -> int:
    desc = prefill_desc(q, k, v, gates, out)
    params = make_params(top_k, window, block)
    nbytes = ctypes.c_size_t()
    check(lib().nsa_prefill_workspace_bytes(ctypes.byref(desc), ctypes.byref(params), ctypes.byref(nbytes)))
    return nbytes.value


def prefill_general_workspace_bytes(q, k, v, gates, out, *, top_k, window, block=64, select_block=None,
                                     stride=None, compressor=None, gate_layer=None, scale: float = 0.0) -> int:
    desc = prefill_desc(q, k, v, gates if gates is not None else q[..., :3], out)
    params = make_params(top_k, window, block, select_block, scale)
    gen = make_general(block if stride is None else stride, compressor, gate_layer)
    nbytes = ctypes.c_size_t()
    check(lib().nsa_prefill_general_workspace_bytes(ctypes.byref(desc), ctypes.byref(params), ctypes.byref(gen),
                                                    ctypes.byref(nbytes)))
    return nbytes.value


def decode_workspace_bytes(q, k_cache, v_cache, kc_cache, vc_cache, gates, out, *, top_k, window, block=64,
                           select_block=None) -> int:
    desc = decode_desc(q, k_cache, v_cache, kc_cache, vc_cache, gates, out)
    params = make_params(top_k, window, block, select_block)
    nbytes = ctypes.c_size_t()
    check(lib().nsa_decode_workspace_bytes(ctypes.byref(desc), ctypes.byref(params), ctypes.byref(nbytes)))
    return nbytes.value


def prefill_backward_workspace_bytes(q, k, v, gates, dout, *, top_k, window, block=64) -> int:
    desc = prefill_desc(q, k, v, gates, dout)
    params = make_params(top_k, window, block)
    nbytes = ctypes.c_size_t()
    check(lib().nsa_bwd_prefill_workspace_bytes(ctypes.byref(desc), ctypes.byref(params), ctypes.byref(nbytes)))
    return nbytes.value


def prefill_save(q, k, v, gates, *, top_k: int, window: int, block: int = 64, scale: float = 0.0,
                 out_dtype=None, idx=None, inject: bool = False, workspace=None):
    """nsa_fwd_prefill_save: the prefill plus what the backward keeps of the
    selected branch. Returns (out, idx, (o_slc, lse_slc)); with inject=True,
    idx supplies the selection."""
    _require_gpu(q, k, v, gates)
    B, L, Hq, D = q.shape
    G = k.shape[2]
    out = torch.empty((B, L, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    if idx is None:
        if inject:
            raise ValueError("inject=True needs idx")
        idx = torch.empty((B, L, G, top_k), dtype=torch.int32, device=q.device)
    o_slc = torch.empty_like(out)
    lse_slc = torch.empty((B, L, Hq), dtype=torch.float32, device=q.device)
    desc = prefill_desc(q, k, v, gates, out)
    params = make_params(top_k, window, block, scale=scale)
    if workspace is None:
        workspace = torch.empty(prefill_workspace_bytes(q, k, v, gates, out, top_k=top_k, window=window,
                                                        block=block), dtype=torch.uint8, device=q.device)
    check(lib().nsa_fwd_prefill_save(ctypes.byref(desc), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(gates), _ptr(out), _ptr(idx),
                                     NSA_IDX_INJECT if inject else NSA_IDX_COMPUTE, _ptr(o_slc),
                                     _ptr(lse_slc), _ptr(workspace), workspace.numel(), _stream_of(q)))
    return out, idx, (o_slc, lse_slc)


def prefill_backward(q, k, v, gates, dout, idx, *, top_k: int, window: int, block: int = 64,
                     scale: float = 0.0, grads=None, workspace=None, saved=None):
    """Gradients of sum(out * dout) of the NSA prefill for the fixed selection idx.

    q, k, v, gates as for prefill(); dout [B,L,Hq,D] in the output dtype;
    idx [B,L,G,top_k] int32 (the forward's selection). Returns float32
    (dq, dk, dv, dgates); `grads` may supply those four contiguous tensors.
    `saved` = (o_slc, lse_slc) from prefill_save() selects nsa_bwd_prefill_saved.
    """
    _require_gpu(q, k, v, gates, dout, idx)
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 tensor")
    B, L, Hq, D = q.shape
    G = k.shape[2]
    if tuple(idx.shape) != (B, L, G, top_k):
        raise ValueError(f"idx shape {tuple(idx.shape)} != {(B, L, G, top_k)}")
    if grads is None:
        f32 = dict(dtype=torch.float32, device=q.device)
        grads = (torch.empty((B, L, Hq, D), **f32), torch.empty((B, L, G, D), **f32),
                 torch.empty((B, L, G, D), **f32), torch.empty((B, L, Hq, 3), **f32))
    for gtn in grads:
        if gtn.dtype != torch.float32 or not gtn.is_contiguous():
            raise ValueError("gradient outputs must be contiguous float32 tensors")
    desc = prefill_desc(q, k, v, gates, dout)
    params = make_params(top_k, window, block, scale=scale)
    if workspace is None:
        workspace = torch.empty(prefill_backward_workspace_bytes(q, k, v, gates, dout, top_k=top_k,
                                                                 window=window, block=block),
                                dtype=torch.uint8, device=q.device)
    if saved is not None:
        o_slc, lse_slc = saved
        check(lib().nsa_bwd_prefill_saved(ctypes.byref(desc), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(gates), _ptr(dout), _ptr(idx), _ptr(o_slc), _ptr(lse_slc),
                                          *(_ptr(x) for x in grads), _ptr(workspace), workspace.numel(),
                                          _stream_of(q)))
        return grads
    check(lib().nsa_bwd_prefill(ctypes.byref(desc), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(gates),
                                _ptr(dout), _ptr(idx), *(_ptr(x) for x in grads), _ptr(workspace),
                                workspace.numel(), _stream_of(q)))
    return grads


def decode_desc(q, k_cache, v_cache, kc_cache, vc_cache, gates, out) -> DecodeDesc:
    B, Hq, D = q.shape
    _, G, Lmax, _ = k_cache.shape
    d = DecodeDesc()
    d.batch, d.max_seqlen, d.max_blocks = B, Lmax, kc_cache.shape[2]
    d.n_q_heads, d.n_kv_heads, d.head_dim = Hq, G, D
    d.in_dtype, d.out_dtype = _dtype_code(q.dtype), _dtype_code(out.dtype)
    d.q_stride[:] = q.stride()[:2]
    d.k_stride[:] = k_cache.stride()[:3]
    d.v_stride[:] = v_cache.stride()[:3]
    d.kc_stride[:] = kc_cache.stride()[:3]
    d.vc_stride[:] = vc_cache.stride()[:3]
    d.g_stride[:] = gates.stride()[:2]
    d.o_stride[:] = out.stride()[:2]
    return d


def decode(q, k_cache, v_cache, kc_cache, vc_cache, seqlens, gates, *, top_k: int, window: int,
           block: int = 64, select_block=None, scale: float = 0.0, out=None, out_dtype=None,
           idx=None, inject: bool = False, return_idx: bool = False, workspace=None):
    """NSA decode. q [B,Hq,D]; caches [B,G,Lmax,D]; block caches [B,G,Nmax,D];
    seqlens [B] int32 (device); gates [B,Hq,3]. Returns out (and idx [B,G,top_k])."""
    _require_gpu(q, k_cache, v_cache, kc_cache, vc_cache, gates)
    B, Hq, D = q.shape
    G = k_cache.shape[1]
    if seqlens.dtype != torch.int32 or not seqlens.is_cuda or seqlens.shape != (B,):
        raise ValueError("seqlens must be an int32 device tensor of shape [B]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    if inject and idx is None:
        raise ValueError("inject=True needs idx")
    if idx is None and return_idx:
        idx = torch.empty((B, G, top_k), dtype=torch.int32, device=q.device)
    if idx is not None and (idx.dtype != torch.int32 or not idx.is_contiguous()
                            or tuple(idx.shape) != (B, G, top_k)):
        raise ValueError("idx must be a contiguous int32 [B, G, top_k] tensor")
    desc = decode_desc(q, k_cache, v_cache, kc_cache, vc_cache, gates, out)
    params = make_params(top_k, window, block, select_block, scale)
    L_ = lib()
    nbytes = ctypes.c_size_t()
    check(L_.nsa_decode_workspace_bytes(ctypes.byref(desc), ctypes.byref(params), ctypes.byref(nbytes)))
    if workspace is None or workspace.numel() < nbytes.value:
        workspace = torch.empty(max(nbytes.value, 1), dtype=torch.uint8, device=q.device)
    check(L_.nsa_fwd_decode(ctypes.byref(desc), ctypes.byref(params), _ptr(q), _ptr(k_cache),
                            _ptr(v_cache), _ptr(kc_cache), _ptr(vc_cache), _ptr(seqlens),
                            _ptr(gates), _ptr(out), _ptr(idx),
                            NSA_IDX_INJECT if inject else NSA_IDX_COMPUTE, _ptr(workspace),
                            workspace.numel(), _stream_of(q)))
    if idx is not None:
        return out, idx
    return out


def decode_general(q, k_cache, v_cache, kc_cache, vc_cache, seqlens, gates, *, top_k: int, window: int,
                   block: int = 64, select_block=None, stride=None, gate_layer=None, scale: float = 0.0,
                   out=None, out_dtype=None, idx=None, inject: bool = False, return_idx: bool = False,
                   workspace=None):
    """NSA decode with the general geometry (nsa_fwd_decode_general): the
    block caches hold the representations of the blocks [i*stride,
    i*stride + block) of each sequence; selection blocks of select_block
    tokens; a gate layer (gate_w [Hq,D,3], gate_b [Hq,3]), with which gates
    may be None."""
    tensors = [q, k_cache, v_cache, kc_cache, vc_cache] + ([gates] if gates is not None else [])
    _require_gpu(*tensors)
    B, Hq, D = q.shape
    G = k_cache.shape[1]
    if seqlens.dtype != torch.int32 or not seqlens.is_cuda or seqlens.shape != (B,):
        raise ValueError("seqlens must be an int32 device tensor of shape [B]")
    if gates is None and gate_layer is None:
        raise ValueError("gates are needed unless a gate layer computes them")
    for t in list(gate_layer or ()):
        if t.dtype != q.dtype:
            raise TypeError("the gate layer must share the inputs' dtype")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    if inject and idx is None:
        raise ValueError("inject=True needs idx")
    if idx is None and return_idx:
        idx = torch.empty((B, G, top_k), dtype=torch.int32, device=q.device)
    if idx is not None and (idx.dtype != torch.int32 or not idx.is_contiguous()
                            or tuple(idx.shape) != (B, G, top_k)):
        raise ValueError("idx must be a contiguous int32 [B, G, top_k] tensor")
    desc = decode_desc(q, k_cache, v_cache, kc_cache, vc_cache, gates if gates is not None else q[..., :3], out)
    params = make_params(top_k, window, block, select_block, scale)
    gen = make_general(block if stride is None else stride, None, gate_layer)
    L_ = lib()
    nbytes = ctypes.c_size_t()
    check(L_.nsa_decode_general_workspace_bytes(ctypes.byref(desc), ctypes.byref(params), ctypes.byref(gen),
                                                ctypes.byref(nbytes)))
    if workspace is None or workspace.numel() < nbytes.value:
        workspace = torch.empty(max(nbytes.value, 1), dtype=torch.uint8, device=q.device)
    check(L_.nsa_fwd_decode_general(ctypes.byref(desc), ctypes.byref(params), ctypes.byref(gen), _ptr(q),
                                    _ptr(k_cache), _ptr(v_cache), _ptr(kc_cache), _ptr(vc_cache), _ptr(seqlens),
                                    _ptr(gates), _ptr(out), _ptr(idx),
                                    NSA_IDX_INJECT if inject else NSA_IDX_COMPUTE, _ptr(workspace),
                                    workspace.numel(), _stream_of(q)))
    if idx is not None:
        return out, idx
    return out


def decode_noalloc(q, k_cache, v_cache, kc_cache, vc_cache, seqlens, gates, *, top_k: int, window: int,
                   out, idx=None, inject: bool = False, block: int = 64, select_block=None, scale: float = 0.0):
    """nsa_fwd_decode_noalloc: the decode with the library's own device
    scratch (no workspace). out (and idx) must be given, so that nothing is
    allocated on this path either."""
    _require_gpu(q, k_cache, v_cache, kc_cache, vc_cache, gates, out)
    B, Hq, D = q.shape
    G = k_cache.shape[1]
    if seqlens.dtype != torch.int32 or not seqlens.is_cuda or seqlens.shape != (B,):
        raise ValueError("seqlens must be an int32 device tensor of shape [B]")
    if inject and idx is None:
        raise ValueError("inject=True needs idx")
    if idx is not None and (idx.dtype != torch.int32 or not idx.is_contiguous()
                            or tuple(idx.shape) != (B, G, top_k)):
        raise ValueError("idx must be a contiguous int32 [B, G, top_k] tensor")
    desc = decode_desc(q, k_cache, v_cache, kc_cache, vc_cache, gates, out)
    params = make_params(top_k, window, block, select_block, scale)
    check(lib().nsa_fwd_decode_noalloc(ctypes.byref(desc), ctypes.byref(params), _ptr(q), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(kc_cache), _ptr(vc_cache), _ptr(seqlens), _ptr(gates),
                                       _ptr(out), _ptr(idx), NSA_IDX_INJECT if inject else NSA_IDX_COMPUTE,
                                       _stream_of(q)))
    return (out, idx) if idx is not None else out


def compress_kv(k, v, kc=None, vc=None, *, block: int = 64):
    """Block means of a [B,G,L,D] K/V cache -> kc, vc [B,G,L//block,D] (or given tensors)."""
    _require_gpu(k, v)
    B, G, L, D = k.shape
    nc = L // block
    if kc is None:
        kc = torch.empty((B, G, nc, D), dtype=k.dtype, device=k.device)
    if vc is None:
        vc = torch.empty((B, G, nc, D), dtype=v.dtype, device=v.device)
    arr = lambda t: (c_i64 * 3)(*t.stride()[:3])
    check(lib().nsa_compress_kv(B, G, L, D, _dtype_code(k.dtype), block, _ptr(k), arr(k), _ptr(v),
                                arr(v), _ptr(kc), arr(kc), _ptr(vc), arr(vc), _stream_of(k)))
    return kc, vc


def dsa_desc(q, k, v, qi, ki, w, out) -> DsaDesc:
    B, L, Hq, D = q.shape
    d = DsaDesc()
    d.batch, d.seqlen, d.n_q_heads, d.n_kv_heads, d.head_dim = B, L, Hq, k.shape[2], D
    d.idx_heads, d.idx_dim = qi.shape[2], qi.shape[3]
    d.in_dtype, d.out_dtype = _dtype_code(q.dtype), _dtype_code(out.dtype)
    d.q_stride[:] = q.stride()[:3]
    d.k_stride[:] = k.stride()[:3]
    d.v_stride[:] = v.stride()[:3]
    d.o_stride[:] = out.stride()[:3]
    d.qi_stride[:] = qi.stride()[:3]
    d.ki_stride[:] = ki.stride()[:2]
    d.w_stride[:] = w.stride()[:2]
    return d


def dsa_workspace_bytes(q, k, v, qi, ki, w, out, *, top_k: int) -> int:
    n = ctypes.c_size_t()
    check(lib().nsa_dsa_workspace_bytes(ctypes.byref(dsa_desc(q, k, v, qi, ki, w, out)),
                                        ctypes.byref(DsaParams(top_k, 0.0)), ctypes.byref(n)))
    return n.value


def dsa_prefill(q, k, v, qi, ki, w, *, top_k: int, scale: float = 0.0, out=None, out_dtype=None, idx=None,
                inject: bool = False, return_idx: bool = False, workspace=None):
    """Token-level sparse attention with a ReLU indexer (nsa_dsa_prefill).
    q [B,L,Hq,D], k/v [B,L,G,D], qi [B,L,Hi,Di], ki [B,L,Di], w [B,L,Hi].
    Returns out (and idx [B,L,top_k] int32 when return_idx or idx is given)."""
    _require_gpu(q, k, v, qi, ki, w)
    B, L, Hq, D = q.shape
    G = k.shape[2]
    Hi, Di = qi.shape[2], qi.shape[3]
    if (k.shape != (B, L, G, D) or v.shape != k.shape or qi.shape[:2] != (B, L) or ki.shape != (B, L, Di)
            or w.shape != (B, L, Hi)):
        raise ValueError("shape mismatch among q, k, v, qi, ki, w")
    if not (q.dtype == k.dtype == v.dtype == qi.dtype == ki.dtype == w.dtype):
        raise TypeError("all inputs must share one dtype")
    if out is None:
        out = torch.empty((B, L, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    if inject and idx is None:
        raise ValueError("inject=True needs idx")
    if idx is None and return_idx:
        idx = torch.empty((B, L, top_k), dtype=torch.int32, device=q.device)
    if idx is not None and (idx.dtype != torch.int32 or not idx.is_contiguous()
                            or tuple(idx.shape) != (B, L, top_k)):
        raise ValueError("idx must be a contiguous int32 [B, L, top_k] tensor")
    desc = dsa_desc(q, k, v, qi, ki, w, out)
    params = DsaParams(top_k, scale)
    L_ = lib()
    nbytes = ctypes.c_size_t()
    check(L_.nsa_dsa_workspace_bytes(ctypes.byref(desc), ctypes.byref(params), ctypes.byref(nbytes)))
    if workspace is None or workspace.numel() < nbytes.value:
        workspace = torch.empty(max(nbytes.value, 1), dtype=torch.uint8, device=q.device)
    check(L_.nsa_dsa_prefill(ctypes.byref(desc), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(qi), _ptr(ki),
                             _ptr(w), _ptr(out), _ptr(idx), NSA_IDX_INJECT if inject else NSA_IDX_COMPUTE,
                             _ptr(workspace), workspace.numel(), _stream_of(q)))
    if idx is not None:
        return out, idx
    return out
