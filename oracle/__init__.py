"""Float64 CPU oracle of the NSA forward pass (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package; the GPU library never does.
"""
from .nsa_ref import compress, decode, nsa_token, prefill, select_blocks, softmax_attend

__all__ = ["compress", "decode", "nsa_token", "prefill", "select_blocks", "softmax_attend"]
