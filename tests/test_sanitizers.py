"""The CPU oracle and the host side of the C ABI, built with AddressSanitizer
and UndefinedBehaviorSanitizer, run clean.

The pages order the device work by stream alone (glm_spec.rs,
glm5_verify_rows and glm5_verify_rollback docs), so the race and memory
checks that can run here are on the host code: the oracle (every entry point
over small cases, exact-size buffers, 1 and several threads) and the ABI's
validation (every entry point accepted and refused, the kernel launchers
replaced by recording stubs, two threads refusing at once).  Both are built
with gcc/g++ for the host only; no GPU code is involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)   # the sanitizer runtime must come first
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert out.returncode == 0 and out.stdout.strip().endswith("OK"), out.stdout + out.stderr
    assert "runtime error" not in out.stderr and "ERROR: AddressSanitizer" not in out.stderr, \
        out.stderr


def test_oracle_under_asan_and_ubsan(tmp_path):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no gcc")
    exe = tmp_path / "oracle_driver"
    subprocess.run([cc, "-std=c11", *SAN, "-ffp-contract=off", "-pthread",
                    os.path.join(ROOT, "oracle", "kda_oracle.c"),
                    os.path.join(HERE, "oracle_driver.c"), "-o", str(exe), "-lm"], check=True)
    _run(exe)


def test_abi_validation_under_asan_and_ubsan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.isdir(os.path.join(ROCM_INCLUDE, "hip")):
        pytest.skip("no g++ or no HIP headers")
    exe = tmp_path / "abi_driver"
    subprocess.run([cxx, "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE,
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "gated_delta_rule_rows_amd", "csrc"),
                    os.path.join(ROOT, "gated_delta_rule_rows_amd", "csrc", "kda_abi.cpp"),
                    os.path.join(HERE, "abi_driver.cpp"), "-o", str(exe), "-pthread"],
                   check=True)
    _run(exe)
