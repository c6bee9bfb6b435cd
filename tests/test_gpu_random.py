"""Randomised GPU parity: many small shapes (ragged S, both head dimensions,
both masks, random scales including negative and large ones, peaked inputs),
each through the single-pass and the split-KV entry points, compared element
by element with the fp64 oracle. The case list is drawn from a fixed seed, so
the test is deterministic.
"""
import numpy as np
import pytest

import oracle
from parity import compare, gpu_available, run_gpu
from testkit import make_qkv

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _cases(n=24, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([64, 128]))
        S = int(rng.integers(1, 700))
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        causal = bool(rng.integers(0, 2))
        mult = float(rng.choice([1.0, 1.0, 3.0]))
        if rng.random() < 0.5:
            scale = float(np.float32(1.0 / np.sqrt(D)))
        else:
            scale = float(np.float32(rng.uniform(-1.0, 1.0)))
        n_splits = int(rng.integers(1, 9))
        out.append((B, H, S, D, causal, scale, mult, n_splits, 1000 + i))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "B{}H{}S{}D{}{}s{:.3f}x{}n{}".format(
    c[0], c[1], c[2], c[3], "c" if c[4] else "n", c[5], c[6], c[7]))
def test_random_shape(case):
    import torch

    import exact_attention_forward_05_amd as attn

    B, H, S, D, causal, scale, mult, n_splits, seed = case
    print(f"[gpu-random] {case}", flush=True)
    q, k, v = make_qkv(B, H, S, D, seed, qk_mult=mult)
    O, L = oracle.sdpa_forward(q, k, v, scale, causal)
    o, l = run_gpu(q, k, v, scale, causal)
    compare(o, l, O, L, f"single pass {case}")
    dev = torch.device("cuda:0")
    qt, kt, vt = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    os_, ls_ = attn.fwd_splitkv(qt, kt, vt, n_splits=n_splits, scale=scale, causal=causal)
    torch.cuda.synchronize()
    compare(os_.cpu().numpy(), ls_.cpu().numpy(), O, L, f"split-KV {case}")


def _long_cases(n=8, seed=20261203):
    """Shapes from 2048 keys with ragged lengths, both masks and random
    scales: at D = 64 the three-wave geometry (192-key intervals, tails in
    any of the three phases; split runs keep two waves when causal), at
    D = 128 the ping-pong order; long rows whose max keeps climbing exercise
    the lazy-max redo."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        S = int(rng.integers(2048, 9000))
        H = int(rng.integers(1, 3))
        causal = bool(i % 2)
        scale = float(np.float32(0.125)) if rng.random() < 0.5 else float(
            np.float32(rng.uniform(-0.5, 0.5)))
        mult = float(rng.choice([1.0, 3.0]))
        n_splits = int(rng.integers(1, 5))
        out.append((1, H, S, 64, causal, scale, mult, n_splits, 2000 + i))
    rng = np.random.default_rng(seed + 1)
    for i in range(n // 2 + 2):
        S = int(rng.integers(2048, 6000))
        causal = bool(i % 2)
        scale = float(np.float32(128 ** -0.5)) if rng.random() < 0.5 else float(
            np.float32(rng.uniform(-0.4, 0.4)))
        mult = float(rng.choice([1.0, 3.0]))
        n_splits = int(rng.integers(1, 5))
        out.append((1, int(rng.integers(1, 3)), S, 128, causal, scale, mult, n_splits, 2100 + i))
    return out


@pytest.mark.parametrize("case", _long_cases(), ids=lambda c: "B{}H{}S{}D{}{}s{:.3f}x{}n{}".format(
    c[0], c[1], c[2], c[3], "c" if c[4] else "n", c[5], c[6], c[7]))
def test_random_long_shape(case):
    test_random_shape(case)


def _extreme_cases(n=40, seed=20261205):
    """Random shapes with scales up to 6 in magnitude and Q, K up to 3x wider:
    scores spanning hundreds of log2 units, so a row's probabilities are one
    key's or a few keys' (the lazy max redoes often, most probabilities
    vanish). A third of the cases run as S_q < S_k caches."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        Sk = int(rng.integers(1, 2600))
        cache = rng.random() < 0.33
        if cache:
            Sq = int(rng.integers(1, min(Sk, 300) + 1)) if causal else int(rng.integers(1, 300))
        else:
            Sq = Sk
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        mult = float(rng.choice([1.0, 2.0, 3.0]))
        scale = float(np.float32(rng.uniform(-6.0, 6.0)))
        n_splits = int(rng.integers(1, 17))
        out.append((B, H, Sq, Sk, D, causal, scale, mult, n_splits, 5000 + i))
    return out


@pytest.mark.parametrize("case", _extreme_cases(), ids=lambda c: "B{}H{}q{}k{}D{}{}s{:.2f}x{}n{}".format(
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "n", c[6], c[7], c[8]))
def test_random_extreme_scales(case):
    import torch

    import exact_attention_forward_05_amd as attn

    B, H, Sq, Sk, D, causal, scale, mult, n_splits, seed = case
    print(f"[gpu-random] extreme {case}", flush=True)
    q, _, _ = make_qkv(B, H, Sq, D, seed, qk_mult=mult)
    _, k, v = make_qkv(B, H, Sk, D, seed + 7919, qk_mult=mult)
    O, L = oracle.sdpa_forward(q, k, v, scale, causal)
    dev = torch.device("cuda:0")
    qt, kt, vt = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    runs = [("kvcache", attn.fwd_kvcache(qt, kt, vt, n_splits=n_splits, scale=scale,
                                         causal=causal))]
    if Sq == Sk:
        runs.append(("single pass", attn.fwd(qt, kt, vt, scale=scale, causal=causal)))
        runs.append(("split-KV", attn.fwd_splitkv(qt, kt, vt, n_splits=n_splits, scale=scale,
                                                  causal=causal)))
    torch.cuda.synchronize()
    for tag, (o, l) in runs:
        compare(o.cpu().numpy(), l.cpu().numpy(), O, L, f"{tag} {case}")
