"""The bench's one-line JSON contract on the GPU: a short run of bench.py as
a child process (the timed steps only) must print the metric line with the
fields and types the harness reads, a roofline object for the launched
kernel and the parity of the GPU output against the oracle."""
import json
import os
import subprocess
import sys

import pytest

from parity import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_contract():
    print("[gpu-bench] short bench run", flush=True)
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--no-sweep", "--steps", "20",
           "--warmup", "2", "--prewarm-ms", "50", "--clock-seconds", "0", "--gemm-seconds", "0",
           "--cpu-sample-rows", "64"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    line = res.stdout.strip().splitlines()[-1]
    d = json.loads(line)
    assert d["metric"] and d["unit"] == "TFLOP/s" and d["value"] > 0
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 2
    assert d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["scaling"] in ("weak", "strong") and d["vs_baseline"] is None
    assert d["dtype"] == "f16" and d["data"] == "synthetic"
    assert d["config"]["workload"] == "sdpa_b1h8s4096d64"
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert 0 < r["achieved"] < r["peak"] and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["kernel"].startswith("attn_fwd_kernel<64,false,false,")
    assert r["sclk_mhz"] is None and r["gemm_reference_tflops"] is None  # both switched off
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert d["parity"]["pass"] is True
