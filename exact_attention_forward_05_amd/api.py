"""Torch-facing binding of the attention forward library.

torch supplies device memory and the stream; every step of the computation runs
in the HIP kernels behind the C ABI.
"""
from __future__ import annotations

import functools
import heapq
import math
from typing import Optional, Tuple, Union

import torch

from . import _lib


def default_scale(D: int) -> float:
    """1/sqrt(D), the usual scaled-dot-product default."""
    return 1.0 / math.sqrt(D)


def _prepare(q, k, v, scale, out, lse, stream):
    """Checks and output allocation shared by the entry points."""
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
    return B, H, S, D, float(scale), out, lse, stream


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
        causal: bool = False, out: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None,
        stream: Optional[torch.cuda.Stream] = None,
        variant: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Exact attention forward on the GPU.

    q, k, v: fp16 CUDA tensors of one shape [B, H, S, D], contiguous, D in {64, 128}.
    Returns (o, lse): o fp16 [B, H, S, D] and lse fp32 [B, H, S] (natural log).
    ``out``/``lse`` may be preallocated. The call is asynchronous on ``stream``
    (default: torch's current stream). ``variant`` selects a compiled kernel
    variant (``_lib.VARIANT_*``; 0 is the default kernel).

    One workgroup folds each 128-row query tile, so a problem with fewer
    tiles than the GPU has CUs (B*H*ceil(S/128) < 256 on MI355X), or a causal
    one whose longest tiles dominate, leaves CUs idle: :func:`fwd_splitkv`
    with ``n_splits="auto"`` spreads the keys over more workgroups there.
    """
    B, H, S, D, scale, out, lse, stream = _prepare(q, k, v, scale, out, lse, stream)
    with torch.cuda.device(q.device):
        if variant:
            st = _lib.attn_fwd_variant(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       lse.data_ptr(), B, H, S, D, scale, int(bool(causal)),
                                       int(variant), stream.cuda_stream)
        else:
            st = _lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr(), B, H, S, D, scale, int(bool(causal)),
                               stream.cuda_stream)
    _lib.check(st)
    return out, lse


BLOCK_M = 128     # query rows per workgroup
PAIR_KEYS = 128   # keys per tile pair (two 64-key tiles)
# Per-interval time (one tile pair per wave), fixed work per query tile (Q
# load, first copies, epilogue; in intervals), and the combine's HBM rate and
# fixed cost. Fitted to split-KV timings of causal B1 H8 S4096/S8192 D64,
# B1 H2 S8192 D128, B1 H4 S4096 D128 and B2 H4 S2048 D64 at 1-6 runs on
# MI355X (sustained clock); only the choice between split counts depends on
# them (the chosen count was within 1.5% of the fastest on those shapes).
_INTERVAL_US = {64: 1.05, 128: 1.6}
_TILE_FIXED = 1.0
_COMBINE_GBS = 4000.0
_COMBINE_FIXED_US = 3.0
_SPLIT_CHOICES = (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64)


def _intervals_per_tile(Sq: int, Sk: int, causal: bool) -> list:
    """Key intervals (of PAIR_KEYS keys) each query tile folds: all of S_k, or
    (causal; queries at positions S_k - S_q + i) the keys up to the tile's
    last query."""
    n_qt = -(-Sq // BLOCK_M)
    n_all = -(-Sk // PAIR_KEYS)
    if not causal:
        return [n_all] * n_qt
    off = Sk - Sq
    return [-(-min(Sk, BLOCK_M * (t + 1) + off) // PAIR_KEYS) for t in range(n_qt)]


@functools.lru_cache(maxsize=256)
def _workgroup_costs(B: int, H: int, S: int, causal: bool, s: int, n_cus: int,
                     Sk: Optional[int] = None) -> list:
    """Cost of every workgroup of a launch with ``s`` runs (one pass when
    s == 1), in key intervals plus a fixed cost per query tile that a
    workgroup loads, following the kernel's work orders: each query tile's
    intervals are cut into ``s`` runs; a causal single pass folds mirror
    pairs of tiles (two tiles loaded) when that still fills the CUs. ``S`` is
    the query length, ``Sk`` the key length (default ``S``)."""
    Sk = S if Sk is None else Sk
    n_qt = -(-S // BLOCK_M)
    pairs = _intervals_per_tile(S, Sk, causal)
    costs = []
    if s == 1 and causal and B * H * ((n_qt + 1) // 2) >= n_cus:
        for u in range((n_qt + 1) // 2):
            a = n_qt - 1 - u
            costs.append(pairs[a] + _TILE_FIXED if u == a
                         else pairs[a] + pairs[u] + 2 * _TILE_FIXED)
    else:
        for p in pairs:
            for r in range(s):
                costs.append((r + 1) * p // s - r * p // s + _TILE_FIXED)
    return costs * (B * H)


def choose_splits(B: int, H: int, S: int, D: int, causal: bool, n_cus: int = 256,
                  Sk: Optional[int] = None) -> int:
    """Split count for attn_fwd_splitkv from a small cost model.

    Each workgroup (one per CU: the registers of its waves -- eight, two per
    SIMD, or at D = 64 twelve, three per SIMD -- and at D = 128 its 136 KB of
    LDS leave room for no second)
    costs its run of
    tile pairs plus a fixed cost per query tile it loads
    (:func:`_workgroup_costs`); workgroups are placed in launch order, largest
    first, on the least loaded CU; a split count above one adds the partial
    results' HBM traffic and a second launch. Returns the cheapest count.
    """
    n_qt = -(-S // BLOCK_M)
    if B * H * n_qt >= 4 * n_cus and not causal:
        return 1
    longest = max(_intervals_per_tile(S, S if Sk is None else Sk, causal))
    best, best_us = 1, math.inf
    for s in _SPLIT_CHOICES:
        if s > max(1, longest):  # never more runs than the longest tile has intervals
            break
        costs = sorted(_workgroup_costs(B, H, S, causal, s, n_cus, Sk), reverse=True)
        if len(costs) > 200000:
            break
        loads = [0.0] * min(n_cus, len(costs))
        heapq.heapify(loads)
        for c in costs:
            heapq.heapreplace(loads, loads[0] + c)
        us = max(loads) * _INTERVAL_US[D]
        if s > 1:
            rows = B * H * S
            nbytes = 2 * s * rows * (D + 1) * 4 + rows * (D * 2 + 4)
            us += nbytes / (_COMBINE_GBS * 1e3) + _COMBINE_FIXED_US
        if us < best_us:
            best, best_us = s, us
    return best


def fwd_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                n_splits: Union[int, str] = "auto", scale: Optional[float] = None,
                causal: bool = False, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-KV attention forward: each query tile's keys are cut into
    ``n_splits`` runs folded by separate workgroups, then merged by a combine
    kernel. Same arguments and results as :func:`fwd`, plus ``n_splits``
    ("auto" = :func:`choose_splits`) and an optional uint8 ``workspace`` of at
    least ``splitkv_workspace_size`` bytes (allocated here when omitted).
    """
    B, H, S, D, scale, out, lse, stream = _prepare(q, k, v, scale, out, lse, stream)
    if n_splits == "auto":
        n_splits = choose_splits(B, H, S, D, bool(causal),
                                 torch.cuda.get_device_properties(q.device).multi_processor_count)
    n_splits = int(n_splits)
    need = _lib.splitkv_workspace_size(B, H, S, D, n_splits)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        if not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous CUDA tensor on q's device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        st = _lib.attn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), B, H, S, D, scale, int(bool(causal)),
                                   n_splits, ws_ptr, ws_bytes, stream.cuda_stream)
    _lib.check(st)
    return out, lse


def fwd_kvcache(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                n_splits: Union[int, str] = "auto", scale: Optional[float] = None,
                causal: bool = False, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Queries against a key/value cache: q [B, H, S_q, D], k and v
    [B, H, S_k, D] (fp16, contiguous, one device). The queries are the last
    S_q positions, so ``causal`` hides from query i the keys after position
    S_k - S_q + i (needs S_q <= S_k). Returns (o [B, H, S_q, D] fp16, lse
    [B, H, S_q] fp32). Split-KV over the keys (``n_splits``, "auto" =
    :func:`choose_splits`), with an optional uint8 ``workspace``.
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA tensor")
        if t.dtype != torch.float16 or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D float16 tensor")
    if k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError(f"q [B,H,S_q,D] and k, v [B,H,S_k,D] expected: "
                         f"{tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if q.device != k.device or q.device != v.device:
        raise ValueError("q, k, v must be on one device")
    B, H, Sq, D = (int(x) for x in q.shape)
    Sk = int(k.shape[2])
    if scale is None:
        scale = default_scale(D)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.float16 or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous fp16 tensor shaped like q on q's device")
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, H, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous fp32 tensor [B,H,S_q] on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    if n_splits == "auto":
        n_splits = choose_splits(B, H, Sq, D, bool(causal),
                                 torch.cuda.get_device_properties(q.device).multi_processor_count,
                                 Sk=Sk)
    n_splits = int(n_splits)
    need = _lib.splitkv_workspace_size(B, H, Sq, D, n_splits)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        if not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous CUDA tensor on q's device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        st = _lib.attn_fwd_kvcache(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), B, H, Sq, Sk, D, float(scale),
                                   int(bool(causal)), n_splits, ws_ptr, ws_bytes,
                                   stream.cuda_stream)
    _lib.check(st)
    return out, lse
