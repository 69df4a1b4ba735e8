"""MI355X-native Native Sparse Attention (NSA) forward: libnsa (HIP, gfx950) + binding."""
from .nsa import NsaError, compress_kv, decode, prefill  # noqa: F401

__all__ = ["NsaError", "compress_kv", "decode", "prefill"]
