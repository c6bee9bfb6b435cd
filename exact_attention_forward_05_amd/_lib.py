"""ctypes binding of the C ABI declared in include/attn_fwd.h.

Argument marshalling only: the library does all of the work on the GPU. If the
library has not been built, loading raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattn_fwd.so")

ATTN_OK = 0
MAX_SPLITS = 64  # ATTN_MAX_SPLITS
STATUS_NAMES = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_UNSUPPORTED",
                4: "ATTN_ERR_ALIGN", 5: "ATTN_ERR_ARG", 6: "ATTN_ERR_HIP"}

# (name, restype, argtypes) of every exported entry point
_SIGNATURES = [
    ("attn_fwd", ctypes.c_int,
     [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
      ctypes.c_void_p]),
    ("attn_fwd_splitkv", ctypes.c_int,
     [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
      ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    ("attn_fwd_kvcache", ctypes.c_int,
     [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
      ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    ("attn_fwd_variant", ctypes.c_int,
     [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
      ctypes.c_int, ctypes.c_void_p]),
    ("attn_fwd_splitkv_noalloc", ctypes.c_int,
     [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
      ctypes.c_int, ctypes.c_void_p]),
    ("attn_fwd_splitkv_workspace_size", ctypes.c_size_t,
     [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    ("attn_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("attn_last_error", ctypes.c_char_p, []),
    ("attn_version", ctypes.c_int, []),
]

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


def load() -> ctypes.CDLL:
    """Load libattn_fwd.so (once). Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -m exact_attention_forward_05_amd.build` "
                "(the attention path has no CPU fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, res, args in _SIGNATURES:
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int) -> None:
    if status != ATTN_OK:
        raise AttnError(status, load().attn_last_error().decode(errors="replace"))


def attn_fwd(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int,
             S: int, D: int, scale: float, causal: int, stream: int) -> int:
    """Raw call of the C entry point with integer addresses; returns the status."""
    return load().attn_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, S, D,
                           ctypes.c_float(scale), causal, stream)


def attn_fwd_kvcache(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int,
                     S_q: int, S_k: int, D: int, scale: float, causal: int, n_splits: int,
                     ws_ptr: int, ws_bytes: int, stream: int) -> int:
    """Raw call of the key/value-cache entry point; returns the status."""
    return load().attn_fwd_kvcache(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, S_q, S_k, D,
                                   ctypes.c_float(scale), causal, n_splits, ws_ptr, ws_bytes,
                                   stream)


# Kernel variants (ATTN_VARIANT_*) and the head dimensions each is built for.
VARIANT_DEFAULT, VARIANT_RING3, VARIANT_EXP_POLY, VARIANT_WIDE = 0, 1, 2, 4
VARIANT_SUBPIPE, VARIANT_SYNC, VARIANT_BAR2, VARIANT_PROD, VARIANT_TRIO = 8, 16, 32, 64, 128
VARIANT_QUAD = 256
VARIANT_ROT = 512
VARIANT_M32 = 1024
VARIANTS = {64: (0, 1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 1152), 128: (0, 2, 16)}


def attn_fwd_variant(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int,
                     S: int, D: int, scale: float, causal: int, variant: int, stream: int) -> int:
    """Raw call of the variant entry point with integer addresses; returns the status."""
    return load().attn_fwd_variant(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, S, D,
                                   ctypes.c_float(scale), causal, variant, stream)


def attn_fwd_splitkv(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int,
                     S: int, D: int, scale: float, causal: int, n_splits: int, ws_ptr: int,
                     ws_bytes: int, stream: int) -> int:
    """Raw call of the split-KV entry point with integer addresses; returns the status."""
    return load().attn_fwd_splitkv(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, S, D,
                                   ctypes.c_float(scale), causal, n_splits, ws_ptr, ws_bytes,
                                   stream)


def attn_fwd_splitkv_noalloc(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int,
                             H: int, S: int, D: int, scale: float, causal: int, n_splits: int,
                             stream: int) -> int:
    """Raw call of the allocation-free split-KV entry point; returns the status."""
    return load().attn_fwd_splitkv_noalloc(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, S, D,
                                           ctypes.c_float(scale), causal, n_splits, stream)


NOALLOC_SCRATCH_BYTES = 32 << 20  # ATTN_NOALLOC_SCRATCH_BYTES


def splitkv_workspace_size(B: int, H: int, S: int, D: int, n_splits: int) -> int:
    """Bytes of workspace attn_fwd_splitkv needs (0 for n_splits == 1 or bad arguments)."""
    return int(load().attn_fwd_splitkv_workspace_size(B, H, S, D, n_splits))
