"""GPU parity of the launch shapes that select each workgroup order
(csrc/work_order.h), compared element by element with the fp64 oracle:
head-major non-causal launches whose workgroup count is not a multiple of the
8 XCDs, causal launches folded into mirror tile pairs (odd tile counts, whose
middle tile runs alone; ragged sequence tails; head counts not a multiple of
8), and causal launches on either side of the folding threshold (256 folded
workgroups)."""
import numpy as np
import pytest

import oracle
from parity import compare, gpu_available, run_gpu
from testkit import make_qkv

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

CASES = [
    # B, H, S, D, causal, what
    (3, 7, 700, 128, False, "head-major, 126 workgroups (126 % 8 = 6)"),
    (1, 13, 800, 64, False, "head-major, 91 workgroups (91 % 8 = 3), ragged tail"),
    (1, 64, 1100, 64, True, "folded, 9 tiles: middle tile alone, ragged tail"),
    (2, 37, 1300, 128, True, "folded, 11 tiles, 444 workgroups (444 % 8 = 4)"),
    (2, 64, 512, 128, True, "folded at the threshold: 256 workgroups"),
    (1, 85, 768, 64, True, "one tile per workgroup just below it: 255 folded"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}S{}D{}{}".format(
    c[0], c[1], c[2], c[3], "c" if c[4] else "n"))
def test_work_order_shapes_full_compare(case):
    B, H, S, D, causal, what = case
    print(f"[gpu-work-order] {case}", flush=True)
    q, k, v = make_qkv(B, H, S, D, 5100 + B * 1000 + H)
    scale = 1.0 / np.sqrt(D)
    o, l = run_gpu(q, k, v, scale, causal)
    O, L = oracle.sdpa_forward(q, k, v, scale, causal)
    compare(o, l, O, L, what)
