"""GPU parity of every compiled kernel variant (attn_fwd_variant) against the
fp64 oracle, element by element over the whole output: the three-slot K/V
ring, the 64-row waves and the sub-tile pipelined interval at D = 64, the
exponential offload and the synchronous-copy check at both head dimensions. Shapes span several tiles with ragged tails, both masks, B > 1,
negative and large scales, and rows whose running max moves mid-sequence."""
import math

import numpy as np
import pytest

import oracle
from parity import compare, gpu_available
from testkit import WORKLOADS, make_qkv, workload_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

# (D, variant) pairs built into the library, besides the default kernel
BUILT = [(64, 1), (64, 2), (64, 4), (64, 8), (64, 16), (64, 32), (64, 64), (64, 128),
         (64, 256), (64, 512), (64, 1024), (64, 1152), (128, 2), (128, 16)]
NAMES = {1: "ring3", 2: "exp_poly", 4: "wide", 8: "subpipe", 16: "sync", 32: "bar2",
         64: "prod", 128: "trio", 256: "quad", 512: "rot", 1024: "m32", 1152: "m32_trio"}

SHAPES = [
    # B, H, S, causal, scale, seed
    (1, 2, 17, False, 0.125, 1),
    (2, 3, 300, True, 0.125, 2),
    (1, 2, 640, True, -0.2, 3),
    (1, 1, 1000, False, 0.5, 4),
    (3, 2, 385, False, None, 5),
    (2, 1, 1, True, 0.3, 6),          # one key: every tile masked past the first key
]


def run_variant(q, k, v, scale, causal, variant):
    import torch

    import exact_attention_forward_05_amd as attn

    dev = torch.device("cuda:0")
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v))
    o, lse = attn.fwd(qt, kt, vt, scale=scale, causal=causal, variant=variant)
    torch.cuda.synchronize(dev)
    return o.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("D,variant", BUILT, ids=[f"D{d}-{NAMES[v]}" for d, v in BUILT])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda c: "B{}H{}S{}{}".format(
    c[0], c[1], c[2], "c" if c[3] else "n"))
def test_variant_small_shapes_full_compare(D, variant, shape):
    B, H, S, causal, scale, seed = shape
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    print(f"[gpu-variants] D{D} {NAMES[variant]} {shape}", flush=True)
    q, k, v = make_qkv(B, H, S, D, 9500 + seed + D)
    o, l = run_variant(q, k, v, scale, causal, variant)
    O, L = oracle.sdpa_forward(q, k, v, scale, causal)
    compare(o, l, O, L, f"D{D} {NAMES[variant]} {shape}")


@pytest.mark.parametrize("D,variant", BUILT, ids=[f"D{d}-{NAMES[v]}" for d, v in BUILT])
def test_variant_running_max_moves(D, variant):
    """Peaked rows next to flat rows (Q x 4 / x 1/2 per 16-row half) and keys
    scaled by 4 mid-sequence, both masks: the lazy max refreshes in some
    sub-tiles only."""
    for causal in (False, True):
        q, k, v = make_qkv(1, 2, 700, D, 9600 + D + variant)
        rows = np.arange(700)
        q = q.astype(np.float32)
        q[:, :, (rows % 32) < 16, :] *= 4.0
        q[:, :, (rows % 32) >= 16, :] *= 0.5
        k = k.astype(np.float32)
        k[:, :, [200, 450, 601], :] *= 4.0
        q, k = q.astype(np.float16), k.astype(np.float16)
        scale = float(np.float32(1.0 / math.sqrt(D)))
        o, l = run_variant(q, k, v, scale, causal, variant)
        O, L = oracle.sdpa_forward(q, k, v, scale, causal)
        compare(o, l, O, L, f"lazy max D{D} {NAMES[variant]} causal={causal}")


@pytest.mark.parametrize("variant", [1, 2, 4, 512, 1024, 1152], ids=lambda v: NAMES[v])
def test_variant_headline_full_compare(variant):
    w = WORKLOADS["sdpa_b1h8s4096d64"]
    q, k, v = workload_inputs(w)
    o, l = run_variant(q, k, v, w.scale, w.causal, variant)
    O, L = oracle.sdpa_forward(q, k, v, w.scale, w.causal)
    print(f"[gpu-variants] headline {NAMES[variant]} "
          f"{compare(o, l, O, L, f'headline {NAMES[variant]}')}", flush=True)


@pytest.mark.parametrize("variant", [1024, 1152], ids=lambda v: NAMES[v])
@pytest.mark.parametrize("causal,scale,mult", [(True, 0.125, 1.0), (True, -0.3, 3.0),
                                               (False, 1.0, 1.0)],
                         ids=["causal", "causal_peaked_negative", "noncausal_scale1"])
def test_m32_long_rows(variant, causal, scale, mult):
    """32x32x16 MFMAs over 2500 keys (a ragged tail in the three-wave
    geometry's 192-key intervals), with the causal diagonal, peaked and
    negative-scale scores."""
    print(f"[gpu-variants] {NAMES[variant]} S2500 causal={causal} scale={scale} x{mult}",
          flush=True)
    q, k, v = make_qkv(1, 2, 2500, 64, 9650 + variant % 7, qk_mult=mult)
    o, l = run_variant(q, k, v, scale, causal, variant)
    O, L = oracle.sdpa_forward(q, k, v, scale, causal)
    compare(o, l, O, L, f"{NAMES[variant]} S2500 causal={causal} scale={scale}")


def test_exp_poly_peaked_causal_d128():
    """The exponential offload at D = 128 on a slice of the peaked causal
    workload (Q, K x 3): 8 heads of S = 4096, every row compared."""
    w = WORKLOADS["peaked_causal_b4h32s4096d128"]
    q, k, v = (x[:1, :8] for x in workload_inputs(w))
    q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
    o, l = run_variant(q, k, v, w.scale, True, 2)
    O, L = oracle.sdpa_forward(q, k, v, w.scale, True)
    print(f"[gpu-variants] peaked D128 exp_poly {compare(o, l, O, L, 'peaked exp_poly')}",
          flush=True)


def test_unbuilt_variant_is_refused():
    import torch

    import exact_attention_forward_05_amd as attn

    q = torch.zeros((1, 1, 64, 128), dtype=torch.float16, device="cuda:0")
    with pytest.raises(attn.AttnError, match="ATTN_ERR_UNSUPPORTED"):
        attn.fwd(q, q, q, variant=1)


SYNC_SHAPES = [
    # B, H, S, D, causal: tails, both masks, folded causal pairs (256 workgroups
    # after folding), two rounds per XCD with the backwards key order
    (2, 3, 300, 64, True),
    (1, 2, 1000, 64, False),
    (1, 16, 4096, 64, True),
    (1, 64, 1024, 64, False),
    # causal three waves per SIMD: tiles not folded; folded from 8192 keys
    (1, 8, 4096, 64, True),
    (1, 8, 8192, 64, True),
    (2, 3, 300, 128, True),
    (1, 2, 1000, 128, False),
    (1, 16, 4096, 128, True),
    (1, 64, 1024, 128, False),
]


@pytest.mark.parametrize("shape", SYNC_SHAPES, ids=lambda c: "B{}H{}S{}D{}{}".format(
    c[0], c[1], c[2], c[3], "c" if c[4] else "n"))
def test_synchronous_copies_equal_the_default_bitwise(shape):
    """The ring-protocol check: with every copy waited for and barriered right
    after its issue (and D = 128 in lock-step), the results must equal the
    default kernel's bit for bit; a read of a ring slot before its copy lands,
    or a copy over a slot still being read, would show here."""
    B, H, S, D, causal = shape
    print(f"[gpu-variants] sync vs default {shape}", flush=True)
    q, k, v = make_qkv(B, H, S, D, 9800 + S + D)
    scale = D ** -0.5
    o0, l0 = run_variant(q, k, v, scale, causal, 0)
    o1, l1 = run_variant(q, k, v, scale, causal, 16)
    assert np.array_equal(o0.view(np.uint16), o1.view(np.uint16)), f"{shape}: O differs"
    assert np.array_equal(l0.view(np.uint32), l1.view(np.uint32)), f"{shape}: LSE differs"
