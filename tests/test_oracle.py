"""Pins for the CPU oracle, each against something other than the oracle itself.

Every check takes the attention function under test as an argument, so the
same checks also run against oracles with planted mistakes (see
``test_planted_mistakes_are_caught``): each plausible mistake must fail at
least one check.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oa
from testkit import WORKLOADS, make_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _t(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64))


# --------------------------------------------------------------------------
# checks (each raises AssertionError on failure)
# --------------------------------------------------------------------------

def check_bruteforce(sdpa):
    """Pure-Python evaluation without max subtraction, exp and fsum in fp64."""
    for causal in (False, True):
        q, k, v = make_qkv(2, 2, 5, 3, 101)
        scale = 0.6875
        O, L = sdpa(q, k, v, scale, causal)
        qf, kf, vf = (x.astype(float).tolist() for x in (q, k, v))
        for b in range(2):
            for h in range(2):
                for i in range(5):
                    js = range(i + 1) if causal else range(5)
                    w = {j: math.exp(scale * math.fsum(qf[b][h][i][d] * kf[b][h][j][d]
                                                       for d in range(3))) for j in js}
                    z = math.fsum(w.values())
                    for d in range(3):
                        ref = math.fsum(w[j] * vf[b][h][j][d] for j in js) / z
                        assert abs(O[b, h, i, d] - ref) <= 1e-12, (b, h, i, d)
                    assert abs(L[b, h, i] - math.log(z)) <= 1e-12


def check_torch_sdpa(sdpa):
    """torch's scaled_dot_product_attention in float64 on the CPU, and
    torch.logsumexp of explicitly formed masked scores for the LSE."""
    for (B, H, S, D, causal, scale) in [(2, 3, 37, 16, False, 0.25),
                                        (2, 3, 37, 16, True, 0.25),
                                        (1, 2, 70, 8, True, 1.3125)]:
        q, k, v = make_qkv(B, H, S, D, 202 + S)
        O, L = sdpa(q, k, v, scale, causal)
        ref = torch.nn.functional.scaled_dot_product_attention(
            _t(q), _t(k), _t(v), is_causal=causal, scale=scale)
        assert np.abs(O - ref.numpy()).max() <= 1e-12
        s = scale * torch.matmul(_t(q), _t(k).transpose(-1, -2).contiguous())
        if causal:
            s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), -math.inf)
        assert np.abs(L - torch.logsumexp(s, dim=-1).numpy()).max() <= 1e-12


def check_rows_sum_to_one(sdpa):
    """V = identity makes O_i the softmax row itself: non-negative, sums to 1."""
    for causal in (False, True):
        q, k, _ = make_qkv(1, 2, 8, 8, 303)
        v = np.broadcast_to(np.eye(8, dtype=np.float16), (1, 2, 8, 8)).copy()
        O, _ = sdpa(q, k, v, 0.5, causal)
        assert O.min() >= 0.0
        assert np.abs(O.sum(-1) - 1.0).max() <= 1e-12
        if causal:
            assert np.abs(np.triu(O[0, 0], 1)).max() == 0.0


def check_constant_v(sdpa):
    for causal in (False, True):
        q, k, v = make_qkv(2, 2, 19, 8, 404)
        v[:] = v[:, :, :1, :]
        O, _ = sdpa(q, k, v, 0.40625, causal)
        ref = np.broadcast_to(v[:, :, :1, :].astype(np.float64), O.shape)
        assert np.abs(O - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def check_equal_scores(sdpa):
    """scale = 0 or Q = 0: O_i is the mean of the visible V rows and
    LSE_i = ln |J_i| (ln S, or ln(i+1) when causal)."""
    S = 23
    for causal in (False, True):
        for mode in ("scale0", "q0"):
            q, k, v = make_qkv(1, 2, S, 8, 505)
            scale = 0.0 if mode == "scale0" else 0.90625
            if mode == "q0":
                q[:] = 0
            O, L = sdpa(q, k, v, scale, causal)
            vf = v.astype(np.float64)
            for i in range(S):
                n = i + 1 if causal else S
                assert np.abs(O[:, :, i] - vf[:, :, :n].mean(axis=2)).max() <= 1e-12
                assert np.abs(L[:, :, i] - math.log(n)).max() <= 1e-12


def check_causal_row0(sdpa):
    q, k, v = make_qkv(2, 3, 17, 8, 606)
    O, L = sdpa(q, k, v, 0.625, True)
    assert np.abs(O[:, :, 0] - v[:, :, 0].astype(np.float64)).max() == 0.0
    s00 = 0.625 * np.einsum("bhd,bhd->bh", q[:, :, 0].astype(np.float64),
                          k[:, :, 0].astype(np.float64))
    assert np.abs(L[:, :, 0] - s00).max() <= 1e-12


def check_single_key(sdpa):
    for causal in (False, True):
        q, k, v = make_qkv(2, 2, 1, 16, 707)
        O, L = sdpa(q, k, v, 0.3125, causal)
        assert np.abs(O - v.astype(np.float64)).max() == 0.0
        s = 0.3125 * (q.astype(np.float64) * k.astype(np.float64)).sum(-1)
        assert np.abs(L - s).max() <= 1e-12


def check_permutation(sdpa):
    q, k, v = make_qkv(1, 2, 29, 8, 808)
    O, L = sdpa(q, k, v, 0.5, False)
    rng = np.random.default_rng(0)
    pk = rng.permutation(29)
    O2, L2 = sdpa(q, k[:, :, pk], v[:, :, pk], 0.5, False)
    assert np.abs(O2 - O).max() <= 1e-12 and np.abs(L2 - L).max() <= 1e-12
    pq = rng.permutation(29)
    O3, L3 = sdpa(q[:, :, pq], k, v, 0.5, False)
    assert np.abs(O3 - O[:, :, pq]).max() <= 1e-12
    assert np.abs(L3 - L[:, :, pq]).max() <= 1e-12


def check_bounds(sdpa):
    for causal in (False, True):
        q, k, v = make_qkv(1, 3, 31, 8, 909, qk_mult=2.0)
        scale = 0.34375
        O, L = sdpa(q, k, v, scale, causal)
        vf = v.astype(np.float64)
        s = scale * np.einsum("bhid,bhjd->bhij", q.astype(np.float64), k.astype(np.float64))
        for i in range(31):
            n = i + 1 if causal else 31
            lo = vf[:, :, :n].min(axis=2)
            hi = vf[:, :, :n].max(axis=2)
            assert (O[:, :, i] >= lo - 1e-12).all() and (O[:, :, i] <= hi + 1e-12).all()
            m = s[:, :, i, :n].max(axis=-1)
            assert (L[:, :, i] >= m - 1e-12).all()
            assert (L[:, :, i] <= m + math.log(n) + 1e-12).all()


def check_last_row(sdpa):
    q, k, v = make_qkv(2, 2, 21, 8, 1010)
    Oc, Lc = sdpa(q, k, v, 0.5, True)
    On, Ln = sdpa(q, k, v, 0.5, False)
    assert np.abs(Oc[:, :, -1] - On[:, :, -1]).max() <= 1e-12
    assert np.abs(Lc[:, :, -1] - Ln[:, :, -1]).max() <= 1e-12
    assert np.abs(Oc[:, :, :-1] - On[:, :, :-1]).max() > 1e-3


def check_one_hot(sdpa):
    """K rows are basis vectors and q_i = 60 e_{j*(i)} with scale 1: the weight
    of every other key is e^-60 of the chosen one, so O_i = v_{j*(i)} and
    LSE_i = 60 to well below 1e-12."""
    S = D = 16
    _, _, v = make_qkv(1, 1, S, D, 1111)
    k = np.eye(S, dtype=np.float16)[None, None]
    target = (np.arange(S) * 7 + 3) % S
    q = np.zeros((1, 1, S, D), dtype=np.float16)
    q[0, 0, np.arange(S), target] = 60.0
    O, L = sdpa(q, k, v, 1.0, False)
    assert np.abs(O[0, 0] - v[0, 0, target].astype(np.float64)).max() <= 1e-12
    assert np.abs(L[0, 0] - 60.0).max() <= 1e-12


def check_geometric_closed_form(sdpa):
    """Scores in arithmetic progression s_j = t j make the softmax weights a
    truncated geometric distribution with ratio r = e^t. With V rows (j, 1):

      LSE over n keys = ln((r^n - 1) / (r - 1))
      O[0] = E[j] = r/(1-r) - n r^n / (1 - r^n),  O[1] = 1.

    All query rows are equal, so under causal masking row i sees n = i + 1 keys.
    """
    S, D = 12, 4
    a, scale = 0.125, 0.8125
    q = np.zeros((1, 1, S, D), dtype=np.float16)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, S, D), dtype=np.float16)
    k[0, 0, :, 0] = a * np.arange(S)
    v = np.zeros((1, 1, S, D), dtype=np.float16)
    v[0, 0, :, 0] = np.arange(S)
    v[0, 0, :, 1] = 1.0
    t = float(np.float32(scale)) * a
    r = math.exp(t)
    for causal in (False, True):
        O, L = sdpa(q, k, v, scale, causal)
        for i in range(S):
            n = i + 1 if causal else S
            if n == 1:
                mean, lse = 0.0, 0.0
            else:
                mean = r / (1 - r) - n * r**n / (1 - r**n)
                lse = math.log((r**n - 1) / (r - 1))
            assert abs(O[0, 0, i, 0] - mean) <= 1e-12
            assert abs(O[0, 0, i, 1] - 1.0) <= 1e-12
            assert abs(O[0, 0, i, 2:]).max() == 0.0
            assert abs(L[0, 0, i] - lse) <= 1e-12


# ---- queries against a longer key/value cache (S_q < S_k) ----------------

def check_cache_bruteforce(sdpa):
    """Pure-Python fp64 evaluation with S_q != S_k: query i sits at position
    S_k - S_q + i, so under causal masking it sees keys 0 .. S_k - S_q + i."""
    Sq, Sk, D = 3, 7, 4
    q, _, _ = make_qkv(2, 2, Sq, D, 1601)
    _, k, v = make_qkv(2, 2, Sk, D, 1602)
    scale = 0.59375
    for causal in (False, True):
        O, L = sdpa(q, k, v, scale, causal)
        assert O.shape == (2, 2, Sq, D) and L.shape == (2, 2, Sq)
        qf, kf, vf = (x.astype(float).tolist() for x in (q, k, v))
        for b in range(2):
            for h in range(2):
                for i in range(Sq):
                    js = range(Sk - Sq + i + 1) if causal else range(Sk)
                    w = {j: math.exp(scale * math.fsum(qf[b][h][i][d] * kf[b][h][j][d]
                                                       for d in range(D))) for j in js}
                    z = math.fsum(w.values())
                    for d in range(D):
                        ref = math.fsum(w[j] * vf[b][h][j][d] for j in js) / z
                        assert abs(O[b, h, i, d] - ref) <= 1e-12, (b, h, i, d)
                    assert abs(L[b, h, i] - math.log(z)) <= 1e-12


def check_cache_suffix_of_square(sdpa):
    """The last S_q rows of a square problem (S_k queries against the same K
    and V) are exactly the queries-against-cache result for those S_q rows,
    causal or not. This ties the S_q < S_k case to the square case."""
    S, D = 29, 8
    q, k, v = make_qkv(1, 2, S, D, 1603, qk_mult=2.0)
    for causal in (False, True):
        O, L = sdpa(q, k, v, 0.40625, causal)
        for Sq in (1, 5, S):
            O2, L2 = sdpa(np.ascontiguousarray(q[:, :, S - Sq:]), k, v, 0.40625, causal)
            assert np.abs(O2 - O[:, :, S - Sq:]).max() <= 1e-12
            assert np.abs(L2 - L[:, :, S - Sq:]).max() <= 1e-12


def check_cache_torch_mask(sdpa):
    """torch's scaled_dot_product_attention in float64 with the visibility as
    an explicit boolean mask (True = visible), and torch.logsumexp of the
    masked scores."""
    Sq, Sk, D = 11, 40, 16
    q, _, _ = make_qkv(2, 3, Sq, D, 1604)
    _, k, v = make_qkv(2, 3, Sk, D, 1605)
    for causal in (False, True):
        vis = torch.ones(Sq, Sk, dtype=torch.bool)
        if causal:
            vis = torch.arange(Sk)[None, :] <= torch.arange(Sq)[:, None] + (Sk - Sq)
        O, L = sdpa(q, k, v, 0.3125, causal)
        ref = torch.nn.functional.scaled_dot_product_attention(
            _t(q), _t(k), _t(v), attn_mask=vis, scale=0.3125)
        assert np.abs(O - ref.numpy()).max() <= 1e-12
        sc = 0.3125 * torch.matmul(_t(q), _t(k).transpose(-1, -2).contiguous())
        sc = sc.masked_fill(~vis, -math.inf)
        assert np.abs(L - torch.logsumexp(sc, dim=-1).numpy()).max() <= 1e-12


def check_cache_equal_scores(sdpa):
    """scale = 0 with S_q < S_k: O_i is the mean of the visible V rows
    (v_0 .. v_{S_k-S_q+i} when causal, all S_k otherwise) and LSE_i = ln of
    their count."""
    Sq, Sk = 6, 19
    q, _, _ = make_qkv(1, 2, Sq, 8, 1606)
    _, k, v = make_qkv(1, 2, Sk, 8, 1607)
    vf = v.astype(np.float64)
    for causal in (False, True):
        O, L = sdpa(q, k, v, 0.0, causal)
        for i in range(Sq):
            n = Sk - Sq + i + 1 if causal else Sk
            assert np.abs(O[:, :, i] - vf[:, :, :n].mean(axis=2)).max() <= 1e-12
            assert np.abs(L[:, :, i] - math.log(n)).max() <= 1e-12


ALL_CHECKS = [check_bruteforce, check_torch_sdpa, check_rows_sum_to_one, check_constant_v,
              check_equal_scores, check_causal_row0, check_single_key, check_permutation,
              check_bounds, check_last_row, check_one_hot, check_geometric_closed_form,
              check_cache_bruteforce, check_cache_suffix_of_square, check_cache_torch_mask,
              check_cache_equal_scores]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle.sdpa_forward)


# --------------------------------------------------------------------------
# the carrier algebra: partial states over key ranges and their merge
# --------------------------------------------------------------------------

def check_merge(partial, merge):
    for causal in (False, True):
        q, k, v = make_qkv(2, 2, 40, 8, 1212, qk_mult=2.0)
        O, L = oracle.sdpa_forward(q, k, v, 0.5, causal)
        for cuts in ([0, 40], [0, 17, 40], [0, 0, 13, 13, 40], [0, 5, 9, 30, 39, 40]):
            parts = [partial(q, k, v, 0.5, causal, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
            st = parts[0]
            for p in parts[1:]:
                st = merge(st, p)
            O2, L2 = oracle.finalize(st)
            assert np.abs(O2 - O).max() <= 1e-12 and np.abs(L2 - L).max() <= 1e-12
            # merging right-to-left gives the same result (associativity)
            st = parts[-1]
            for p in parts[-2::-1]:
                st = merge(p, st)
            O3, L3 = oracle.finalize(st)
            assert np.abs(O3 - O).max() <= 1e-12 and np.abs(L3 - L).max() <= 1e-12


def test_merge_of_split_key_ranges_equals_unsplit():
    check_merge(oracle.partial_state, oracle.merge_states)


def test_partial_state_identity_for_invisible_ranges():
    q, k, v = make_qkv(1, 1, 10, 4, 1313)
    m, d, o = oracle.partial_state(q, k, v, 0.5, True, 5, 10)
    assert np.isneginf(m[0, 0, :5]).all() and (d[0, 0, :5] == 0).all() and (o[0, 0, :5] == 0).all()
    assert np.isfinite(m[0, 0, 5:]).all()


def test_stream_fold_equals_definition():
    for causal in (False, True):
        q, k, v = make_qkv(2, 2, 33, 8, 1414, qk_mult=3.0)
        O, L = oracle.sdpa_forward(q, k, v, 0.4375, causal)
        O2, L2 = oracle.stream_fold(q, k, v, 0.4375, causal)
        assert np.abs(O2 - O).max() <= 1e-12 and np.abs(L2 - L).max() <= 1e-12


def test_sampled_rows_equal_full_oracle():
    q, k, v = make_qkv(2, 3, 700, 16, 1515)
    O, L = oracle.sdpa_forward(q, k, v, 0.25, True)
    rows = [0, 1, 511, 512, 513, 699]
    O2, L2 = oracle.sdpa_rows(q, k, v, 0.25, True, 1, 2, rows)
    assert np.abs(O2 - O[1, 2, rows]).max() <= 1e-13 and np.abs(L2 - L[1, 2, rows]).max() <= 1e-13


def test_cache_partial_states_and_stream_fold():
    """With S_q < S_k the carriers of split key ranges still merge to the
    unsplit result, and the per-key streaming fold equals the definition."""
    q, _, _ = make_qkv(2, 2, 9, 8, 1608, qk_mult=2.0)
    _, k, v = make_qkv(2, 2, 30, 8, 1609)
    for causal in (False, True):
        O, L = oracle.sdpa_forward(q, k, v, 0.5, causal)
        st = None
        for a, b in ([0, 7], [7, 21], [21, 30]):
            p = oracle.partial_state(q, k, v, 0.5, causal, a, b)
            st = p if st is None else oracle.merge_states(st, p)
        O2, L2 = oracle.finalize(st)
        assert np.abs(O2 - O).max() <= 1e-12 and np.abs(L2 - L).max() <= 1e-12
        O3, L3 = oracle.stream_fold(q, k, v, 0.5, causal)
        assert np.abs(O3 - O).max() <= 1e-12 and np.abs(L3 - L).max() <= 1e-12


def test_cache_shape_checks():
    q, _, _ = make_qkv(1, 2, 9, 8, 1)
    _, k, v = make_qkv(1, 2, 5, 8, 2)
    oracle.sdpa_forward(q, k, v, 0.5, False)          # S_q > S_k is fine without a mask
    with pytest.raises(ValueError):
        oracle.sdpa_forward(q, k, v, 0.5, True)       # causal rows would see no key
    with pytest.raises(ValueError):
        oracle.sdpa_forward(q, k[:, :1], v[:, :1], 0.5, False)  # heads differ


def test_oracle_rejects_non_fp16():
    q, k, v = make_qkv(1, 1, 4, 4, 1)
    with pytest.raises(TypeError):
        oracle.sdpa_forward(q.astype(np.float32), k, v, 0.5)


# --------------------------------------------------------------------------
# the pages' own numbers
# --------------------------------------------------------------------------

def test_pages_workloads_and_flop_convention():
    g = json.load(open(os.path.join(GOLDEN, "pages_workloads.json")))
    p = WORKLOADS["sdpa_b1h8s4096d64"]
    assert list(p.shape) == g["workloads"]["SDPA_P"]["shape"] and not p.causal
    lst = WORKLOADS["listing_b1h4s128d64"]
    assert list(lst.shape) == g["workloads"]["SDPA_L"]["shape"] and not lst.causal
    thr = g["throughput"]
    tflops = p.flops / (thr["latency_us"] * 1e-6) / 1e12
    assert abs(tflops - thr["tflops"]) / thr["tflops"] <= thr["tflops_rel_tol"]
    st = g["listing_strides"]
    q = np.empty(p.shape, dtype=np.float16)
    assert [s // 2 for s in q.strides[:3]] == [st["batch_stride_elems"], st["head_stride_elems"],
                                             st["row_stride_elems"]]


# --------------------------------------------------------------------------
# planted mistakes: each must fail at least one check
# --------------------------------------------------------------------------

def _mutant_rows(kind):
    def rows_of_head(qh, kh, vh, scale, causal, rows):
        S = kh.shape[0]
        off = 0 if kind == "cache_top_left" else S - qh.shape[0]
        if kind == "transposed_qk":
            s = scale * (kh[rows] @ qh.T)
        elif kind == "no_scale":
            s = qh[rows] @ kh.T
        elif kind == "inverse_scale":
            s = (qh[rows] @ kh.T) / scale if scale else qh[rows] @ kh.T
        else:
            s = scale * (qh[rows] @ kh.T)
        j = np.arange(S)[None, :]
        i = rows[:, None] + off
        if causal:
            if kind == "mask_diagonal":
                vis = j < i
            elif kind == "mask_lower":
                vis = j >= i
            else:
                vis = j <= i
            s = np.where(vis, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp2(s - m) if kind == "exp2_base" else np.exp(s - m)
        d = e.sum(axis=1, keepdims=True)
        p = e if kind == "no_normalise" else e / d
        vv = vh[::-1] if kind == "reversed_v" else vh
        o = p @ vv
        if kind == "v_dims_swapped":
            o = o[:, ::-1]
        lse = np.log(d[:, 0]) if kind == "lse_no_max" else m[:, 0] + np.log(d[:, 0])
        if kind == "lse_log2":
            lse = m[:, 0] + np.log2(d[:, 0])
        return o, lse
    return rows_of_head


MUTANTS = ["transposed_qk", "no_scale", "inverse_scale", "mask_diagonal", "mask_lower",
           "exp2_base", "no_normalise", "reversed_v", "v_dims_swapped", "lse_no_max", "lse_log2",
           "cache_top_left"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistakes_are_caught(kind, monkeypatch):
    monkeypatch.setattr(oa, "_rows_of_head", _mutant_rows(kind))
    failed = []
    for check in ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(oa.sdpa_forward)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(check.__name__)
    assert failed, f"no pin caught the planted mistake {kind}"


def test_planted_merge_mistake_is_caught():
    def bad_merge(a, b):
        m1, d1, o1 = a
        m2, d2, o2 = b
        m = np.maximum(m1, m2)
        with np.errstate(invalid="ignore", over="ignore"):
            w1 = np.nan_to_num(np.exp(m - m1))   # sign flipped
            w2 = np.nan_to_num(np.exp(m2 - m))
        return m, d1 * w1 + d2 * w2, o1 * w1[..., None] + o2 * w2[..., None]
    with pytest.raises(AssertionError):
        with np.errstate(all="ignore"):
            check_merge(oracle.partial_state, bad_merge)
