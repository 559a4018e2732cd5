"""Compiles ``libcf.so`` (HIP kernels + C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libcf.so")
SOURCES = ["csrc/cf_api.hip", "csrc/cf_quant.hip", "csrc/cf_lowrank.hip", "csrc/cf_topk.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # one rounding per fp32 operation, in the order written (no FMA contraction)
    "-ffp-contract=off",
    # no packed-fp32 instructions (v_pk_add/mul/fma_f32) in device code.  The feature
    # applies to the gfx950 pass; the x86 host pass does not know it and warns that it
    # ignores it, which is expected.  tests/test_build_flags.py reads the disassembly.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build_library(extra_flags: list[str] | None = None) -> str:
    cmd = [hipcc(), *FLAGS, *(extra_flags or []), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(PKG, "csrc"), *[os.path.join(PKG, s) for s in SOURCES],
           "-o", LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB
