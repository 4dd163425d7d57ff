"""Build the in-tree HIP library ``libgla.so`` for gfx950 with hipcc.

Usage: ``python -m gated_bidirectional_linear_amd.build`` (or ``build()`` from
Python).  Always recompiles; the result lands next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgla.so")
SOURCES = ["gla_tables.hip", "gla_state.hip", "gla_output.hip", "gla_causal.hip", "gla_noalloc.hip", "gla_dispatch.cpp",
           "gla_abi.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def compile_flags() -> list:
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        # no packed-fp32 VALU ops: plain float code only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + compile_flags() + ["-shared", "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libgla.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
