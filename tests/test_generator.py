"""The seeded input generator: determinism, published constants, rounding, moments."""
import math

import numpy as np
import pytest

from testkit import WORKLOADS, make_qkv, normal_f16, normal_f64
from testkit import gen


def test_splitmix64_known_outputs():
    # SplitMix64 seeded with 0 (state advanced by the golden gamma before each
    # output): the first outputs of the published generator.
    expected = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    key = np.uint64(0)
    got = [int(x) for x in gen.raw_draws(key, 0, 3)]
    assert got == expected


def test_streams_are_deterministic_and_distinct():
    a = normal_f64(123, 0, 1000)
    b = normal_f64(123, 0, 1000)
    c = normal_f64(123, 1, 1000)
    d = normal_f64(124, 0, 1000)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)
    assert not np.array_equal(a, d)
    assert abs(np.corrcoef(a, c)[0, 1]) < 0.1


def test_prefix_property_and_chunk_independence():
    # Element i of a stream does not depend on how many elements are drawn.
    n = gen._CHUNK + 1001
    full = normal_f64(5, 2, n)
    assert np.array_equal(full[:77], normal_f64(5, 2, 77))
    h = normal_f16(5, 2, (n,))
    assert np.array_equal(h[:77], normal_f16(5, 2, (77,)))
    assert np.array_equal(h, full.astype(np.float16))


def test_box_muller_pair_layout():
    # Element 2n and 2n+1 come from raw draws 2n, 2n+1 as r cos / r sin.
    key = gen.stream_key(9, 0)
    z = gen.raw_draws(key, 0, 2)
    u1 = ((int(z[0]) >> 11) + 1) * 2.0**-53
    u2 = (int(z[1]) >> 11) * 2.0**-53
    r = math.sqrt(-2.0 * math.log(u1))
    x = normal_f64(9, 0, 2)
    assert x[0] == pytest.approx(r * math.cos(2 * math.pi * u2), rel=1e-15, abs=1e-15)
    assert x[1] == pytest.approx(r * math.sin(2 * math.pi * u2), rel=1e-15, abs=1e-15)


def test_moments_are_standard_normal():
    x = normal_f64(2024, 0, 400_000)
    n = len(x)
    assert abs(x.mean()) < 5 / math.sqrt(n)
    assert abs(x.var() - 1.0) < 5 * math.sqrt(2.0 / n)
    # fourth moment of N(0,1) is 3
    assert abs((x**4).mean() - 3.0) < 0.05
    # tail mass beyond 3 sigma: 0.0027
    assert abs((np.abs(x) > 3).mean() - 0.0027) < 0.0005


def _nearest_f16_rne(x: float) -> np.float16:
    """Nearest fp16 to x by exhaustive neighbour comparison, ties to even."""
    h = np.float16(x)  # candidate, checked below against both neighbours
    cands = {float(h), float(np.nextafter(h, np.float16(np.inf))),
             float(np.nextafter(h, np.float16(-np.inf)))}
    best = min(cands, key=lambda c: (abs(c - x), np.float16(c).view(np.uint16) & 1))
    return np.float16(best)


def test_f16_rounding_is_nearest_even_from_f64():
    x = normal_f64(77, 0, 20000) * 3.0
    h = (x).astype(np.float16)
    for xi, hi in zip(x[:2000], h[:2000]):
        assert float(hi) == float(_nearest_f16_rne(float(xi)))
    # exact ties between two fp16 values round to the even mantissa
    tie = 1.0 + 2.0**-11  # halfway between 1 and 1 + 2^-10
    assert float(np.float16(tie)) == 1.0
    tie2 = 1.0 + 3 * 2.0**-11  # halfway between 1+2^-10 and 1+2^-9
    assert float(np.float16(tie2)) == 1.0 + 2.0**-9
    # a value just above a tie must not be double-rounded through fp32
    above = 1.0 + 2.0**-11 + 2.0**-40
    assert float(np.array([above]).astype(np.float16)[0]) == 1.0 + 2.0**-10


def test_mult_scales_before_the_single_rounding():
    x = normal_f64(31, 1, 1000)
    h = normal_f16(31, 1, (1000,), 3.0)
    assert np.array_equal(h, (3.0 * x).astype(np.float16))


def test_workload_tensors_use_streams_0_1_2():
    q, k, v = make_qkv(1, 2, 8, 4, 11)
    assert q.dtype == np.float16 and q.shape == (1, 2, 8, 4)
    assert np.array_equal(q.reshape(-1), normal_f16(11, 0, (64,)))
    assert np.array_equal(k.reshape(-1), normal_f16(11, 1, (64,)))
    assert np.array_equal(v.reshape(-1), normal_f16(11, 2, (64,)))


def test_workload_table():
    w = WORKLOADS["sdpa_b1h8s4096d64"]
    assert w.shape == (1, 8, 4096, 64) and not w.causal and w.scale == 0.125
    c = WORKLOADS["causal_b2h16s8192d128"]
    assert c.causal and c.scale == float(np.float32(1 / math.sqrt(128)))
    p = WORKLOADS["peaked_causal_b4h32s4096d128"]
    assert p.qk_mult == 3.0 and p.v_mult == 1.0 and p.causal
    seeds = {w.seed for w in WORKLOADS.values()}
    assert len(seeds) == len(WORKLOADS)
