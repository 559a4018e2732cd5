"""The gfx950 code in libcf.so holds no packed fp32 arithmetic.

The build passes ``-Xclang -target-feature -Xclang -packed-fp32-ops`` to hipcc, which
turns off the packed fp32 instructions (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32) for
the device pass; the host pass does not know the feature and says so in a warning, which
is harmless.  This test reads the disassembly of the library's device code objects, as
built here, and checks that none of those instructions is in it (and that the matrix
instructions of the low-rank kernels are, so the disassembly is real).
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "activation_residual_compression_cf_amd", "libcf.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _tool(name):
    path = os.path.join(LLVM, name)
    return path if os.path.exists(path) else shutil.which(name)


def _device_asm(tmp) -> str:
    objcopy, bundler, objdump = _tool("llvm-objcopy"), _tool("clang-offload-bundler"), _tool("llvm-objdump")
    if not (objcopy and bundler and objdump) or not os.path.exists(LIB):
        pytest.skip("ROCm LLVM tools or libcf.so not available")
    fatbin = os.path.join(tmp, "fatbin")
    subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fatbin}", LIB, os.path.join(tmp, "stripped")],
                   check=True, capture_output=True)
    data = open(fatbin, "rb").read()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)] + [len(data)]
    assert len(starts) > 1, "no offload bundle in .hip_fatbin"
    asm = []
    for j, (a, b) in enumerate(zip(starts, starts[1:])):
        bundle, co = os.path.join(tmp, f"b{j}"), os.path.join(tmp, f"b{j}.co")
        with open(bundle, "wb") as f:
            f.write(data[a:b])
        subprocess.run([bundler, "--unbundle", "--type=o", f"--input={bundle}",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"],
                       check=True, capture_output=True)
        asm.append(subprocess.run([objdump, "-d", "--mcpu=gfx950", co], check=True, capture_output=True,
                                  text=True).stdout)
    return "\n".join(asm)


def test_no_packed_fp32_in_device_code(tmp_path):
    asm = _device_asm(str(tmp_path))
    packed = sorted(set(re.findall(r"\bv_pk_(?:add|mul|fma)_f32\b", asm)))
    assert not packed, f"packed fp32 instructions in libcf.so: {packed}"
    assert re.search(r"\bv_mfma_f32_16x16x4", asm), "disassembly holds no low-rank MFMA: nothing was read"
