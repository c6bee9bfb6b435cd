"""GPU parity over the whole output of the three large problem configurations:
every head and every row of O and LSE against the fp64 oracle, at the tolerances
of the attention workloads (O max abs 4e-3, O mean abs 5e-4, LSE max abs 1e-3).

The kernels run exactly as the bench launches them (attn_fwd, the same work
orders). The oracle's rows are evaluated on host threads (tests/parity.py,
oracle_full); each row is still the plain definition.
"""
import os
import time

import pytest

from parity import compare, gpu_available, oracle_full, run_gpu
from testkit import WORKLOADS, workload_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

WORKERS = min(16, os.cpu_count() or 1)


@pytest.mark.parametrize("name", ["long_b1h8s16384d64", "causal_b2h16s8192d128",
                                  "peaked_causal_b4h32s4096d128"])
def test_large_workload_every_head_and_row(name):
    w = WORKLOADS[name]
    print(f"[gpu-parity-full] {name}: {w.describe()}", flush=True)
    q, k, v = workload_inputs(w)
    o, l = run_gpu(q, k, v, w.scale, w.causal)
    t0 = time.time()
    O, L = oracle_full(q, k, v, w.scale, w.causal, workers=WORKERS)
    print(f"[gpu-parity-full] {name}: oracle {time.time() - t0:.1f} s on {WORKERS} threads",
          flush=True)
    stats = compare(o, l, O, L, name)
    print(f"[gpu-parity-full] {name}: {stats}", flush=True)
