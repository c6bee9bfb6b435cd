"""Exact fused attention forward for AMD Instinct MI355X (gfx950).

``fwd(q, k, v, scale=None, causal=False) -> (o, lse)`` runs the HIP kernels of
libattn_fwd.so through its C ABI (include/attn_fwd.h); ``fwd_splitkv`` is the
split-KV variant (key runs folded by separate workgroups, then merged);
``fwd_kvcache`` runs S_q queries against a longer key/value cache.
"""
from ._lib import AttnError, LIB_PATH, load, splitkv_workspace_size
from .api import choose_splits, default_scale, fwd, fwd_kvcache, fwd_splitkv

__all__ = ["AttnError", "LIB_PATH", "load", "splitkv_workspace_size", "choose_splits",
           "default_scale", "fwd", "fwd_kvcache", "fwd_splitkv"]
