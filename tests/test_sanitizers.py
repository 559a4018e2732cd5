"""Sanitizer builds of the host code (CPU only).

- The oracle (``oracle/cf_oracle.c``) is built with AddressSanitizer, LeakSanitizer
  and UBSan and driven through every entry point by ``oracle_sanitize.c``.
- The seeded generator (``gen/cfgen.c``) is built the same way, and once more with
  ThreadSanitizer since it fills trajectories from a thread pool (``gen_sanitize.c``).
- libcf's host code (validation and launch set-up) is built with AddressSanitizer
  and UBSan and its validation driven on overflow-prone sizes and pointer ranges by
  ``abi_sanitize.cpp``.  Its valid calls stop at the device check, so it runs only
  where no GPU driver is present.

Any report aborts the driver with a non-zero status.
"""
import os
import shutil
import subprocess

import pytest

from activation_residual_compression_cf_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")

ASAN_UBSAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", TSAN_OPTIONS="halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stderr[-4000:]
    assert run.stdout.strip() == "ok"
    assert "runtime error" not in run.stderr


def _build_and_run(tmp_path, name, sources, flags):
    exe = str(tmp_path / name)
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", *flags, *sources, "-lm", "-lpthread",
           "-o", exe]
    subprocess.run(cmd, check=True, cwd=ROOT, timeout=120)
    _run(exe)


def test_oracle_under_asan_ubsan(tmp_path):
    _build_and_run(tmp_path, "oracle_asan",
                   ["oracle/cf_oracle.c", os.path.join(HERE, "oracle_sanitize.c")], ASAN_UBSAN)


def test_generator_under_asan_ubsan(tmp_path):
    _build_and_run(tmp_path, "gen_asan", ["gen/cfgen.c", os.path.join(HERE, "gen_sanitize.c")],
                   ASAN_UBSAN)


def test_generator_under_tsan(tmp_path):
    _build_and_run(tmp_path, "gen_tsan", ["gen/cfgen.c", os.path.join(HERE, "gen_sanitize.c")],
                   ["-fsanitize=thread"])


@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="valid calls with placeholder pointers would launch on a present GPU")
@pytest.mark.skipif(not os.path.exists(_build.hipcc()), reason="needs hipcc")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_asan")
    csrc = os.path.join(_build.PKG, "csrc")
    # the host pass alone is instrumented: each sanitizer flag follows -Xarch_host
    san = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all"]
    flags = [f for f in _build.FLAGS if f not in ("-shared", "-fPIC", "-O3")]
    cmd = [_build.hipcc(), *flags, "-O1", "-g", *san, "-I", os.path.join(ROOT, "include"), "-I", csrc,
           "-x", "hip", *[os.path.join(_build.PKG, s) for s in _build.SOURCES],
           os.path.join(HERE, "abi_sanitize.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, cwd=ROOT, timeout=600, capture_output=True)
    _run(exe)
