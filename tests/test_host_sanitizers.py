"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
argument checks and launch geometry of the entry points (csrc/plan.h) and the
workgroup -> tile maps (csrc/work_order.h), compiled with the host C++
compiler with both sanitizers and every UBSan finding fatal, then run."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "exact_attention_forward_05_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
@pytest.mark.parametrize("src", ["host_plan_check.cpp", "work_order_check.cpp"])
def test_host_code_under_asan_ubsan(src, tmp_path):
    exe = str(tmp_path / src.replace(".cpp", ""))
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror", *SAN,
                    f"-I{CSRC}", f"-I{INCLUDE}", "-o", exe, os.path.join(HERE, src)],
                   check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok"), res.stdout + res.stderr
    assert "runtime error" not in res.stderr, res.stderr
