"""Host check of the workgroup -> (head, query tile) maps the kernels use
(csrc/work_order.h): compiled with the host C++ compiler and run on the CPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "exact_attention_forward_05_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_work_orders_cover_every_tile_once(tmp_path):
    exe = str(tmp_path / "work_order_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", f"-I{CSRC}", "-o", exe,
                    os.path.join(HERE, "work_order_check.cpp")], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok")
