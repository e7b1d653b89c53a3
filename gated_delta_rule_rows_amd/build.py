"""Build libkda.so (the gfx950 KDA verify-row scan library) with hipcc.

    python -m gated_delta_rule_rows_amd.build

Flags, and why:
  --offload-arch=gfx950      MI355X only; no other code objects.
  -O3 -ffp-contract=off      every fused multiply-add is an explicit fmaf, so
                             no instantiation can contract differently from
                             another (the entry points must agree bit for bit).
  -target-feature -packed-fp32-ops
                             keep the compiler from forming packed FP32 ops.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = [os.path.join(CSRC, "kda_kernels.hip"), os.path.join(CSRC, "kda_abi.cpp")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", INCLUDE,
    "-I", CSRC,
]


def build(out: str = LIB, extra: tuple = ()) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, *SOURCES, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(extra=tuple(sys.argv[1:])))
