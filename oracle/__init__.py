"""Float64 CPU oracles of the NSA forward pass and of token-level sparse
attention (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package; the GPU library never does.
"""
from .nsa_ref import (compress, decode, gates_from_query, n_compressed, nsa_token, prefill, select_blocks,
                      selection_scores, softmax_attend)

__all__ = ["compress", "decode", "gates_from_query", "n_compressed", "nsa_token", "prefill", "select_blocks",
           "selection_scores", "softmax_attend"]
from . import dsa_ref  # noqa: E402,F401
