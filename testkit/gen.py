"""Seeded synthetic inputs: fp16 tensors of i.i.d. normal draws.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and bench. It draws random numbers and rounds them to fp16; it holds none of
the attention arithmetic.

Generator (all published methods, implemented here from their definitions):

* SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014). The n-th output of a stream keyed by ``key`` is
  ``mix64(key + (n + 1) * GAMMA)``; being counter-based, any element can be
  produced independently, so the tensor is generated in parallel chunks and
  the result does not depend on the chunking.
* A stream key is ``mix64(seed + (stream + 1) * GAMMA)``: one SplitMix64 step
  from the seed at counter ``stream + 1``.
* Uniforms: the top 53 bits of a raw draw. ``u1 = (z >> 11 + 1) * 2^-53`` lies in
  (0, 1] so that ``log(u1)`` is finite; ``u2 = (z >> 11) * 2^-53`` lies in [0, 1).
* Normals: Box & Muller (1958). Pair ``n`` uses raw draws ``2n`` and ``2n+1``;
  element ``2n`` is ``r cos(2 pi u2)`` and element ``2n+1`` is ``r sin(2 pi u2)``
  with ``r = sqrt(-2 ln u1)``, all in fp64.
* The fp64 value times ``mult`` is rounded once, directly to fp16 with
  round-to-nearest-even (numpy's float64 -> float16 cast), never through fp32.

The workloads in the attention pages draw Q, K and V with ``torch.randn`` in
fp16 (Learning FlashAttention the Hard Way, Part 2: the SDPA_P and SDPA_L
workload definitions); this generator stands in for it with a documented,
reproducible stream.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 21  # normals per chunk (an even number)


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, stream: int) -> np.uint64:
    """Key of tensor stream ``stream`` under ``seed`` (both < 2^64)."""
    with np.errstate(over="ignore"):
        s = np.array([seed], dtype=np.uint64) + np.uint64(stream + 1) * GAMMA
    return mix64(s)[0]


def raw_draws(key: np.uint64, start: int, count: int) -> np.ndarray:
    """Raw 64-bit draws ``start .. start+count-1`` of the stream ``key``."""
    n = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(key + n * GAMMA)


def _normals_chunk(key: np.uint64, first: int, count: int) -> np.ndarray:
    """fp64 normals ``first .. first+count-1`` (``first`` and ``count`` even)."""
    z = raw_draws(key, first, count)
    u1 = ((z[0::2] >> np.uint64(11)) + np.uint64(1)).astype(np.float64) * 2.0**-53
    u2 = (z[1::2] >> np.uint64(11)).astype(np.float64) * 2.0**-53
    r = np.sqrt(-2.0 * np.log(u1))
    t = (2.0 * np.pi) * u2
    out = np.empty(count, dtype=np.float64)
    out[0::2] = r * np.cos(t)
    out[1::2] = r * np.sin(t)
    return out


def normal_f64(seed: int, stream: int, n: int) -> np.ndarray:
    """First ``n`` fp64 N(0,1) draws of stream ``stream`` under ``seed``."""
    key = stream_key(seed, stream)
    m = n + (n & 1)
    out = np.empty(m, dtype=np.float64)
    for lo in range(0, m, _CHUNK):
        c = min(_CHUNK, m - lo)
        out[lo:lo + c] = _normals_chunk(key, lo, c)
    return out[:n]


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_f16(seed: int, stream: int, shape, mult: float = 1.0) -> np.ndarray:
    """fp16 tensor of ``shape`` holding ``fp16(mult * x)``, x ~ N(0,1) fp64.

    Element ``i`` of the flattened (row-major) tensor is normal draw ``i`` of
    the stream. Chunks are generated on a thread pool; the values do not
    depend on the number of threads.
    """
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    key = stream_key(seed, stream)
    m = n + (n & 1)
    out = np.empty(m, dtype=np.float16)

    def work(lo: int) -> None:
        c = min(_CHUNK, m - lo)
        x = _normals_chunk(key, lo, c)
        if mult != 1.0:
            x = x * float(mult)
        out[lo:lo + c] = x.astype(np.float16)

    starts = list(range(0, m, _CHUNK))
    if len(starts) == 1:
        work(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, starts))
    return out[:n].reshape(shape)
