"""The threaded full-output oracle helper of the GPU parity tests
(tests/parity.py, oracle_full) against the oracle's own sdpa_forward: the same
rows evaluated in another order and grouping give the same values."""
import numpy as np

import oracle
from parity import oracle_full
from testkit import make_qkv


def test_oracle_full_equals_sdpa_forward():
    for (B, H, S, D, causal, scale) in [(2, 3, 300, 64, True, 0.125),
                                        (1, 2, 1100, 128, False, 0.0883883476)]:
        q, k, v = make_qkv(B, H, S, D, 4711 + S)
        O1, L1 = oracle.sdpa_forward(q, k, v, scale, causal)
        O2, L2 = oracle_full(q, k, v, scale, causal, workers=4, row_chunk=256)
        assert np.abs(O1 - O2).max() <= 1e-12
        assert np.abs(L1 - L2).max() <= 1e-12
