"""GPU parity of queries against a key/value cache (attn_fwd_kvcache): S_q
queries per head against S_k keys, the queries being the last S_q positions
(causal masking bottom-right aligned), split over the keys. Every output row
is compared with the fp64 oracle; the square case is compared bit for bit
with the self-attention entry points."""
import math

import numpy as np
import pytest

import oracle
from parity import compare, gpu_available, oracle_full
from testkit import make_qkv

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _cache_inputs(B, H, Sq, Sk, D, seed, qk_mult=1.0):
    q, _, _ = make_qkv(B, H, Sq, D, seed, qk_mult=qk_mult)
    _, k, v = make_qkv(B, H, Sk, D, seed + 1, qk_mult=qk_mult)
    return q, k, v


def _run(q, k, v, scale, causal, n_splits):
    import torch

    import exact_attention_forward_05_amd as attn

    dev = torch.device("cuda:0")
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v))
    o, lse = attn.fwd_kvcache(qt, kt, vt, n_splits=n_splits, scale=scale, causal=causal)
    torch.cuda.synchronize(dev)
    return o.cpu().numpy(), lse.cpu().numpy()


CASES = [
    # B, H, S_q, S_k, D, causal, n_splits, seed
    (1, 8, 1, 131072, 64, False, "auto", 1),
    (1, 8, 1, 131072, 64, True, "auto", 2),
    (2, 4, 16, 32768, 128, True, "auto", 3),
    (1, 4, 128, 131072, 128, False, "auto", 4),
    (1, 4, 128, 65536, 64, True, 64, 5),
    (2, 3, 5, 1000, 64, True, 7, 6),        # ragged S_k, runs of unequal length
    (1, 2, 300, 777, 128, True, 3, 7),      # several query tiles
    (1, 2, 200, 150, 64, False, 2, 8),      # S_q > S_k without a mask
    (3, 2, 1, 1, 128, True, 1, 9),          # one key
    (1, 2, 16, 4096, 64, True, 64, 10),     # more runs than keys for early rows
    # non-causal D = 64 from 2048 keys: three waves per SIMD, key tails
    (1, 2, 300, 5000, 64, False, 1, 11),
    (2, 2, 130, 4100, 64, False, 3, 12),
    # causal single pass at D = 64 from 2048 keys, tiles not folded: three
    # waves per SIMD with the query block at the end of the keys
    (1, 2, 300, 5000, 64, True, 1, 13),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}q{}k{}D{}{}s{}".format(
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "n", c[6]))
def test_kvcache_full_compare(case):
    B, H, Sq, Sk, D, causal, ns, seed = case
    print(f"[gpu-kvcache] {case}", flush=True)
    q, k, v = _cache_inputs(B, H, Sq, Sk, D, 9400 + seed)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    o, l = _run(q, k, v, scale, causal, ns)
    O, L = oracle_full(q, k, v, scale, causal, row_chunk=64)
    print(f"[gpu-kvcache] {compare(o, l, O, L, str(case))}", flush=True)


def test_kvcache_peaked_scores():
    """Q and K drawn three times wider: the running max moves often."""
    q, k, v = _cache_inputs(2, 4, 64, 20000, 128, 9450, qk_mult=3.0)
    scale = float(np.float32(1.0 / math.sqrt(128)))
    o, l = _run(q, k, v, scale, True, "auto")
    O, L = oracle_full(q, k, v, scale, True, row_chunk=64)
    compare(o, l, O, L, "peaked kvcache")


@pytest.mark.parametrize("scale,causal,ns", [(1.0, True, "auto"), (-0.5, False, 16), (2.0, True, 5)],
                         ids=["s1c", "s-0.5n", "s2c"])
def test_kvcache_large_scales(scale, causal, ns):
    """Long caches with scales far above 1/sqrt(D): rows dominated by a few
    keys, redos of the running max in most runs, split runs merged."""
    q, k, v = _cache_inputs(1, 4, 16, 40000, 64, 9470 + int(4 * scale))
    o, l = _run(q, k, v, scale, causal, ns)
    O, L = oracle_full(q, k, v, scale, causal, row_chunk=64)
    print(f"[gpu-kvcache] scale {scale}: {compare(o, l, O, L, f'large scale {scale}')}", flush=True)


def test_decode_row_is_last_row_of_square_problem():
    """One causal query against the cache equals the last row of the square
    causal problem whose last query it is (the bottom-right alignment)."""
    import torch

    import exact_attention_forward_05_amd as attn

    q, k, v = make_qkv(1, 4, 2048, 64, 9460)
    dev = torch.device("cuda:0")
    qt, kt, vt = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    o_full, l_full = attn.fwd(qt, kt, vt, scale=0.125, causal=True)
    o1, l1 = attn.fwd_kvcache(qt[:, :, -1:].contiguous(), kt, vt, n_splits=8, scale=0.125,
                              causal=True)
    torch.cuda.synchronize()
    assert np.abs(o1.cpu().numpy().astype(np.float64)
                  - o_full[:, :, -1:].cpu().numpy()).max() <= 2e-3
    assert np.abs(l1.cpu().numpy() - l_full[:, :, -1:].cpu().numpy()).max() <= 1e-4


def test_square_cache_is_the_self_attention_path_bitwise():
    import torch

    from exact_attention_forward_05_amd import _lib

    B, H, S, D = 2, 3, 700, 128
    q, k, v = make_qkv(B, H, S, D, 9470)
    dev = torch.device("cuda:0")
    qt, kt, vt = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    st = torch.cuda.current_stream(dev).cuda_stream
    outs = []
    for entry, ns in (("splitkv", 1), ("kvcache", 1), ("splitkv", 3), ("kvcache", 3)):
        o = torch.empty_like(qt)
        l = torch.empty((B, H, S), dtype=torch.float32, device=dev)
        need = _lib.splitkv_workspace_size(B, H, S, D, ns)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        if entry == "splitkv":
            rc = _lib.attn_fwd_splitkv(qt.data_ptr(), kt.data_ptr(), vt.data_ptr(), o.data_ptr(),
                                       l.data_ptr(), B, H, S, D, 0.0883883476, 1, ns,
                                       ws.data_ptr(), ws.numel(), st)
        else:
            rc = _lib.attn_fwd_kvcache(qt.data_ptr(), kt.data_ptr(), vt.data_ptr(), o.data_ptr(),
                                       l.data_ptr(), B, H, S, S, D, 0.0883883476, 1, ns,
                                       ws.data_ptr(), ws.numel(), st)
        _lib.check(rc)
        torch.cuda.synchronize(dev)
        outs.append((o.cpu().numpy().view(np.uint16), l.cpu().numpy().view(np.uint32)))
    for a, b in ((0, 1), (2, 3)):
        assert np.array_equal(outs[a][0], outs[b][0]) and np.array_equal(outs[a][1], outs[b][1])


def _random_cases(n=20, seed=20261204):
    """Random cache shapes: S_q from 1 to 400 queries against up to 6000
    keys (S_q <= S_k under the causal mask, any S_q without it), both head
    dimensions, random scales (negative and large ones), Q and K drawn
    wider in some cases, and random or automatic run counts."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        Sk = int(rng.integers(1, 6000))
        Sq = int(rng.integers(1, min(Sk, 400) + 1)) if causal else int(rng.integers(1, 401))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        mult = float(rng.choice([1.0, 1.0, 3.0]))
        scale = (float(np.float32(1.0 / np.sqrt(D))) if rng.random() < 0.5
                 else float(np.float32(rng.uniform(-1.5, 1.5))))
        ns = "auto" if rng.random() < 0.4 else int(rng.integers(1, 33))
        out.append((B, H, Sq, Sk, D, causal, scale, mult, ns, 9700 + i))
    return out


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: "B{}H{}q{}k{}D{}{}s{:.3f}x{}n{}".format(
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "n", c[6], c[7], c[8]))
def test_kvcache_random_shape(case):
    B, H, Sq, Sk, D, causal, scale, mult, ns, seed = case
    print(f"[gpu-kvcache] random {case}", flush=True)
    q, k, v = _cache_inputs(B, H, Sq, Sk, D, seed, qk_mult=mult)
    o, l = _run(q, k, v, scale, causal, ns)
    O, L = oracle_full(q, k, v, scale, causal, row_chunk=64)
    compare(o, l, O, L, f"random kvcache {case}")
