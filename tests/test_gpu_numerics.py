"""GPU parity on numerically adversarial inputs, against the fp64 oracle at the
standard tolerances: very peaked rows (large scales, including negative),
scores that climb by more than the lazy-max bound in every key tile (a redo
in every tile of every row) or fall away after the first tile (probabilities
far below fp16's normal range), and inputs of large magnitude (fp32
accumulation of large products). Lengths from 2048 keys run the three-wave
geometry at D = 64 and the ping-pong order at D = 128."""
import numpy as np
import pytest

import oracle
from parity import compare, gpu_available, run_gpu
from testkit import make_qkv

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

S = 2500


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["n", "c"])
@pytest.mark.parametrize("scale", [1.0, 4.0, -2.0])
def test_peaked_scales(D, causal, scale):
    q, k, v = make_qkv(1, 2, S, D, 5100 + D + int(8 * scale))
    O, L = oracle.sdpa_forward(q, k, v, scale, causal)
    o, l = run_gpu(q, k, v, scale, causal)
    print(f"[gpu-numerics] peaked D{D} causal={causal} scale={scale}: "
          f"{compare(o, l, O, L, f'peaked D{D} {causal} {scale}')}", flush=True)


def _ramp(D, slope, seed):
    """Q rows along e_0 (plus small noise), K_j = slope * j * e_0 (plus noise):
    score j of every row grows linearly with j."""
    q, k, v = make_qkv(1, 2, S, D, seed, qk_mult=0.01)
    q = q.astype(np.float32)
    k = k.astype(np.float32)
    q[..., 0] = 1.0
    k[..., 0] = slope * np.arange(S, dtype=np.float32)[None, None, :]
    return q.astype(np.float16), k.astype(np.float16), v


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["n", "c"])
@pytest.mark.parametrize("direction", [1.0, -1.0], ids=["climbing", "falling"])
def test_monotone_scores(D, causal, direction):
    """Climbing: +0.3 log2 units per key, 20 per 64-key tile, above the 15 that
    the lazy-max test allows, so every tile of every row redoes. Falling: the
    first tile holds each row's max and later probabilities sink far below
    fp16's normal range."""
    scale = D ** -0.5
    slope = direction * 0.3 / (scale * np.log2(np.e))
    q, k, v = _ramp(D, slope, 5200 + D)
    O, L = oracle.sdpa_forward(q, k, v, scale, causal)
    o, l = run_gpu(q, k, v, scale, causal)
    print(f"[gpu-numerics] monotone D{D} causal={causal} dir={direction}: "
          f"{compare(o, l, O, L, f'monotone D{D} {causal} {direction}')}", flush=True)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["n", "c"])
def test_large_magnitude_inputs(D, causal):
    """Q and K around 100 in magnitude (products up to ~10^4, row dot products
    up to ~10^5 in the fp32 accumulators) with a scale that brings the scores
    back to unit spread."""
    q, k, v = make_qkv(1, 2, S, D, 5300 + D, qk_mult=100.0)
    scale = float(np.float32(D ** -0.5 / 1e4))
    O, L = oracle.sdpa_forward(q, k, v, scale, causal)
    o, l = run_gpu(q, k, v, scale, causal)
    print(f"[gpu-numerics] magnitude D{D} causal={causal}: "
          f"{compare(o, l, O, L, f'magnitude D{D} {causal}')}", flush=True)
