"""Host logic of bench.py, without a GPU: the one-GPU contract, the kernel
source hash that ties a profile summary to the kernel, the profile lookup,
and the work counts the roofline divides by."""
import json
import os
import shutil
import subprocess
import sys

import pytest

import bench
from testkit import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    csrc = tmp_path / "exact_attention_forward_05_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.KERNEL_SOURCES:
        shutil.copy(os.path.join(ROOT, "exact_attention_forward_05_amd", "csrc", f), csrc / f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    k = csrc / bench.KERNEL_SOURCES[0]
    text = k.read_text()
    k.write_text("// an added comment\n/* and a block\n comment */\n" + text.replace("\n", "\n\n", 3))
    assert bench.kernel_source_hash() == h0
    changed = text.replace("BLOCK_M = 128;", "BLOCK_M = 64;", 1)
    assert changed != text  # the edit below is a code change
    k.write_text(changed)
    assert bench.kernel_source_hash() != h0


def test_profiled_traffic_lookup(tmp_path, monkeypatch):
    """A summary's traffic is used only for its workload and only while its
    source hash is the current one."""
    csrc = tmp_path / "exact_attention_forward_05_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.KERNEL_SOURCES:
        shutil.copy(os.path.join(ROOT, "exact_attention_forward_05_amd", "csrc", f), csrc / f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.kernel_source_hash()
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"workload": "sdpa_b1h8s4096d64", "source_hash": h, "traffic_bytes_per_launch": 123}
    old = dict(rec, workload="long_b1h8s16384d64", source_hash="0" * 16)
    (prof / "a.md").write_text("text\n```json\n" + json.dumps(rec) + "\n```\n")
    (prof / "b.md").write_text("```json\n" + json.dumps(old) + "\n```\n")
    assert bench.profiled_traffic("sdpa_b1h8s4096d64") == 123
    assert bench.profiled_traffic("long_b1h8s16384d64") is None   # stale hash
    assert bench.profiled_traffic("no_such_workload") is None


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_work_counts(name):
    w = WORKLOADS[name]
    per_head = w.S * (w.S + 1) // 2 if w.causal else w.S * w.S
    assert bench.visible_scores(w) == w.B * w.H * per_head
    full = 4.0 * w.B * w.H * w.S * w.S * w.D
    assert w.flops == (full / 2 if w.causal else full)
    assert w.algorithmic_bytes == 8 * w.B * w.H * w.S * w.D + 4 * w.B * w.H * w.S


def test_configs_are_the_five_problem_shapes():
    """The bench times these five; their shapes, masks, scales and input
    scaling are the problem configurations."""
    import numpy as np

    from testkit import CONFIGS, WORKLOADS

    want = [(1, 4, 128, 64, False, 1.0), (1, 8, 4096, 64, False, 1.0),
            (1, 8, 16384, 64, False, 1.0), (2, 16, 8192, 128, True, 1.0),
            (4, 32, 4096, 128, True, 3.0)]
    got = [(WORKLOADS[n].B, WORKLOADS[n].H, WORKLOADS[n].S, WORKLOADS[n].D, WORKLOADS[n].causal,
            WORKLOADS[n].qk_mult) for n in CONFIGS]
    assert got == want
    for n in CONFIGS:
        w = WORKLOADS[n]
        assert w.scale == float(np.float32(1.0 / np.sqrt(w.D)))


def test_kernel_label_names_the_launched_instantiation():
    """The roofline's kernel label follows the library's geometry choice:
    three waves per SIMD (variant 128) at D = 64 from 2048 keys, folded causal
    pairs from 8192; two waves below and at D = 128."""
    import bench
    from testkit import WORKLOADS

    want = {
        "listing_b1h4s128d64": "attn_fwd_kernel<64,false,false,0>",
        "sdpa_b1h8s4096d64": "attn_fwd_kernel<64,false,false,128>",
        "long_b1h8s16384d64": "attn_fwd_kernel<64,false,false,128>",
        "causal_b2h16s8192d128": "attn_fwd_kernel<128,true,false,0>",
        "peaked_causal_b4h32s4096d128": "attn_fwd_kernel<128,true,false,0>",
        "sweep_causal_b1h8s4096d64": "attn_fwd_kernel<64,true,false,128>",
    }
    for name, label in want.items():
        assert bench.kernel_label(WORKLOADS[name]) == label, name


def test_parse_sclk_reads_each_gpu_clock():
    """The rocm-smi clock lines the bench samples (one line per GPU; the
    current level is the one reported)."""
    text = ("============================ ROCm System Management Interface ============================\n"
            "=================================== Current clock frequencies ===================================\n"
            "GPU[0]\t\t: fclk clock level: 0: (1900Mhz)\n"
            "GPU[0]\t\t: mclk clock level: 0: (1900Mhz)\n"
            "GPU[0]\t\t: sclk clock level: 1: (2098Mhz)\n"
            "GPU[0]\t\t: socclk clock level: 0: (28Mhz)\n")
    assert bench.parse_sclk(text) == {0: 2098}
    two = text + "GPU[1]\t\t: sclk clock level: 1: (1899Mhz)\n"
    assert bench.parse_sclk(two) == {0: 2098, 1: 1899}
    assert bench.parse_sclk("no clocks here") == {}
