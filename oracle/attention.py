"""CPU oracle for the exact attention forward pass (fp64, numpy).

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
bench's CPU-baseline leg may import or run this module. The GPU product path
never calls it, imports nothing from it, and shares no code with it.

What it computes (the plain definition, not the streaming method):

  For fp16 Q of shape [B,H,S_q,D], K and V of shape [B,H,S_k,D] and a softmax
  scale, for every batch b, head h and query row i, with visible keys
  J_i = {0..S_k-1}, or {0..i+S_k-S_q} when causal (the S_q queries are the
  last S_q positions of the sequence; key j is masked when it lies after the
  query's position; the diagonal is visible). With S_q = S_k = S this is
  J_i = {0..i}:

    s_j   = scale * sum_d q_{i,d} k_{j,d}                  (j in J_i)
    m     = max_j s_j
    e_j   = exp(s_j - m),     d = sum_j e_j
    P_ij  = e_j / d
    O_i   = sum_j P_ij v_j
    LSE_i = m + ln d                                       (natural log)

Sources. The operation is scaled dot-product attention on fp16 [B,H,S,D]
tensors with scale 1/sqrt(D) by default (Learning FlashAttention the Hard Way,
Part 2: the workload definitions, and the unfused Move 0 kernels, which write
the scores out, take the row max, the sum of exponentials, and then the
normalised P times V). The error methodology is an fp64 reference over the
identical fp16-rounded operands (the Emmy comments page, on hybrid FP16/FP32
accumulation). Causal masking, the log-sum-exp output and queries against a
longer key/value cache are not on the pages (the Emmy comments name decoding
against a large KV cache); the readings used are: causal hides key j from
query i when j > i + S_k - S_q (query i sits at position S_k - S_q + i, so
with S_q = S_k it is j > i), and LSE is the natural log of sum_j exp(s_j) over
the visible keys, with s already scaled.

Inputs are promoted exactly from fp16 to fp64 and ``scale`` is the fp32 value
the GPU receives, promoted to fp64. Outputs are fp64 and not rounded.

The partial-state functions below compute the carrier (m, d, o) of a key
range: running max m, denominator d = sum exp(s - m) and unnormalised output
o = sum exp(s - m) v (Part 2's introduction and its FA-1 listing, where the
per-key update is m' = max(m, s), alpha = e^(m - m'), p = e^(s - m'),
d <- d alpha + p, o <- o alpha + p v). Two carriers over disjoint key ranges
combine by rescaling both to the larger max, which is what makes the reduction
split-able across key ranges (Part 2's wrap-up and references, on split-KV).
"""
from __future__ import annotations

import numpy as np

__all__ = ["sdpa_forward", "sdpa_rows", "partial_state", "merge_states",
           "finalize", "stream_fold", "ROW_GROUP"]

# Rows of one head evaluated together. This bounds memory only: every row's
# arithmetic is the definition above, independent of the other rows.
ROW_GROUP = 512


def _f64(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype != np.float16:
        raise TypeError(f"oracle inputs are fp16, got {a.dtype}")
    return a.astype(np.float64)


def _check(q, k, v, causal: bool = False):
    """Q [B,H,S_q,D], K and V [B,H,S_k,D]; causal needs S_q <= S_k (else the
    first query rows would see no key)."""
    if q.ndim != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError(f"Q [B,H,S_q,D] and K, V [B,H,S_k,D] expected: {q.shape} {k.shape} {v.shape}")
    if causal and q.shape[2] > k.shape[2]:
        raise ValueError(f"causal attention needs S_q <= S_k: {q.shape[2]} > {k.shape[2]}")


def _visible(rows: np.ndarray, Sk: int, causal: bool, offset: int = 0) -> np.ndarray:
    """Boolean [len(rows), S_k]: key j visible to query row i, i.e. every key,
    or (causal) j <= i + offset with offset = S_k - S_q."""
    j = np.arange(Sk)
    if not causal:
        return np.ones((len(rows), Sk), dtype=bool)
    return j[None, :] <= rows[:, None] + offset


def _rows_of_head(qh, kh, vh, scale: float, causal: bool, rows: np.ndarray):
    """O and LSE (fp64) for the given query rows of one (b, h) head.

    qh is fp64 [S_q, D], kh and vh fp64 [S_k, D]. Steps follow the definition
    in order.
    """
    Sk = kh.shape[0]
    offset = Sk - qh.shape[0]                          # query i sits at position offset + i
    s = scale * (qh[rows] @ kh.T)                      # scores [r, S_k]
    s = np.where(_visible(rows, Sk, causal, offset), s, -np.inf)
    m = s.max(axis=1, keepdims=True)                   # row max
    e = np.exp(s - m)                                  # masked keys -> 0
    d = e.sum(axis=1, keepdims=True)                   # denominator
    p = e / d                                          # softmax rows
    o = p @ vh                                         # P V
    lse = m[:, 0] + np.log(d[:, 0])
    return o, lse


def sdpa_forward(q, k, v, scale: float, causal: bool = False):
    """Full oracle: O fp64 [B,H,S_q,D] and LSE fp64 [B,H,S_q]."""
    _check(q, k, v, causal)
    B, H, S, D = q.shape
    scale = float(np.float32(scale))
    O = np.empty((B, H, S, D), dtype=np.float64)
    L = np.empty((B, H, S), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            qh, kh, vh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h])
            for lo in range(0, S, ROW_GROUP):
                rows = np.arange(lo, min(S, lo + ROW_GROUP))
                O[b, h, rows], L[b, h, rows] = _rows_of_head(qh, kh, vh, scale, causal, rows)
    return O, L


def sdpa_rows(q, k, v, scale: float, causal: bool, b: int, h: int, rows):
    """Oracle O [len(rows), D] and LSE [len(rows)] for chosen rows of head (b, h)."""
    _check(q, k, v, causal)
    rows = np.asarray(rows, dtype=np.int64)
    scale = float(np.float32(scale))
    return _rows_of_head(_f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), scale, causal, rows)


def partial_state(q, k, v, scale: float, causal: bool, key_lo: int, key_hi: int):
    """Carrier (m, d, o) of every query row over keys [key_lo, key_hi).

    m: [B,H,S] running max (-inf where no key of the range is visible),
    d: [B,H,S] sum of exp(s - m), o: [B,H,S,D] sum of exp(s - m) v.
    A row with no visible key gets the identity (-inf, 0, 0).
    """
    _check(q, k, v, causal)
    B, H, S, D = q.shape
    Sk = k.shape[2]
    scale = float(np.float32(scale))
    m = np.full((B, H, S), -np.inf)
    d = np.zeros((B, H, S))
    o = np.zeros((B, H, S, D))
    keys = np.arange(key_lo, key_hi)
    if len(keys) == 0:
        return m, d, o
    rows = np.arange(S)
    vis = _visible(rows, Sk, causal, Sk - S)[:, keys]
    for b in range(B):
        for h in range(H):
            qh, kh, vh = _f64(q[b, h]), _f64(k[b, h, keys]), _f64(v[b, h, keys])
            s = np.where(vis, scale * (qh @ kh.T), -np.inf)
            mh = s.max(axis=1)
            has = np.isfinite(mh)
            e = np.zeros_like(s)
            e[has] = np.exp(s[has] - mh[has, None])
            m[b, h] = mh
            d[b, h] = e.sum(axis=1)
            o[b, h] = e @ vh
    return m, d, o


def merge_states(a, b):
    """Combine carriers of two disjoint key ranges.

    m = max(m1, m2), d = d1 e^(m1-m) + d2 e^(m2-m), o = o1 e^(m1-m) + o2 e^(m2-m).
    The identity (-inf, 0, 0) is neutral on either side.
    """
    m1, d1, o1 = a
    m2, d2, o2 = b
    m = np.maximum(m1, m2)
    fin = np.isfinite(m)
    safe = np.where(fin, m, 0.0)
    w1 = np.where(fin, np.exp(np.where(np.isfinite(m1), m1, -np.inf) - safe), 0.0)
    w2 = np.where(fin, np.exp(np.where(np.isfinite(m2), m2, -np.inf) - safe), 0.0)
    return m, d1 * w1 + d2 * w2, o1 * w1[..., None] + o2 * w2[..., None]


def finalize(state):
    """O = o / d and LSE = m + ln d from a carrier."""
    m, d, o = state
    return o / d[..., None], m + np.log(d)


def stream_fold(q, k, v, scale: float, causal: bool = False):
    """The streaming method itself, one key at a time, in fp64.

    Starting from the identity, key j is folded into every row's carrier with
    m' = max(m, s_j), alpha = e^(m - m'), p = e^(s_j - m'), d <- d alpha + p,
    o <- o alpha + p v_j, m <- m'. Masked keys are skipped. Returns (O, LSE)
    after the deferred normalisation O = o / d. Loops over keys in Python, so
    it is meant for small S.
    """
    _check(q, k, v, causal)
    B, H, S, D = q.shape
    Sk = k.shape[2]
    scale = float(np.float32(scale))
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    m = np.full((B, H, S), -np.inf)
    d = np.zeros((B, H, S))
    o = np.zeros((B, H, S, D))
    rows = np.arange(S)
    for j in range(Sk):
        s = scale * np.einsum("bhid,bhd->bhi", qf, kf[:, :, j, :])
        vis = np.ones(S, dtype=bool) if not causal else (rows + (Sk - S) >= j)
        m_new = np.where(vis, np.maximum(m, s), m)
        with np.errstate(invalid="ignore"):
            alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
        p = np.where(vis, np.exp(s - m_new), 0.0)
        d = d * alpha + p
        o = o * alpha[..., None] + p[..., None] * vf[:, :, j, None, :]
        m = m_new
    return o / d[..., None], m + np.log(d)
