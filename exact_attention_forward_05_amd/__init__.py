"""Exact fused attention forward for AMD Instinct MI355X (gfx950).

``fwd(q, k, v, scale=None, causal=False) -> (o, lse)`` runs the HIP kernels of
libattn_fwd.so through its C ABI (include/attn_fwd.h).
"""
from ._lib import AttnError, LIB_PATH, load
from .api import default_scale, fwd

__all__ = ["AttnError", "LIB_PATH", "load", "default_scale", "fwd"]
