"""Torch-facing binding of the attention forward library.

torch supplies device memory and the stream; every step of the computation runs
in the HIP kernels behind the C ABI.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import torch

from . import _lib


def default_scale(D: int) -> float:
    """1/sqrt(D), the usual scaled-dot-product default."""
    return 1.0 / math.sqrt(D)


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
        causal: bool = False, out: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None,
        stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Exact attention forward on the GPU.

    q, k, v: fp16 CUDA tensors of one shape [B, H, S, D], contiguous, D in {64, 128}.
    Returns (o, lse): o fp16 [B, H, S, D] and lse fp32 [B, H, S] (natural log).
    ``out``/``lse`` may be preallocated. The call is asynchronous on ``stream``
    (default: torch's current stream).
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA tensor")
        if t.dtype != torch.float16:
            raise TypeError(f"{name} must be float16, got {t.dtype}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B,H,S,D], got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if q.device != k.device or q.device != v.device:
        raise ValueError("q, k, v must be on one device")
    B, H, S, D = (int(x) for x in q.shape)
    if scale is None:
        scale = default_scale(D)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.float16 or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous fp16 tensor shaped like q on q's device")
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, H, S) or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous fp32 tensor [B,H,S] on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        st = _lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           lse.data_ptr(), B, H, S, D, float(scale), int(bool(causal)),
                           stream.cuda_stream)
    _lib.check(st)
    return out, lse
