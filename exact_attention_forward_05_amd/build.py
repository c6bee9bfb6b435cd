"""Build the HIP library libattn_fwd.so in-tree for gfx950.

Usage: python -m exact_attention_forward_05_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libattn_fwd.so"
ARCH = "gfx950"

SOURCES = ["attn_fwd.hip"]
HEADERS = ["attn_fwd_kernel.h", "work_order.h", "plan.h"]

# -packed-fp32-ops: hipcc must not form packed fp32 VALU ops from scalar code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def build(verbose: bool = False) -> str:
    """Compile the library; returns its path. Always recompiles."""
    out = os.path.join(PKG, LIB_NAME)
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), *FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
