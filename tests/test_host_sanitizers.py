"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs are built with g++/gcc (host code only: no GPU code is built
with a sanitizer) and run:

- the C ABI's argument validation (block_quantized_amd/csrc/qmm.cpp) with
  the kernel launchers replaced by counting stand-ins, driven through every
  entry point with valid arguments and each class of invalid one (null,
  misaligned, bad or overflowing sizes, unknown or unsupported types); a
  call that fails validation must launch nothing.  Source: page "The GGML
  ecosystem, and where synapse fits", section 7 (untrusted input is
  validated and rejected, never approximated);
- every function of the CPU oracle on small inputs, edge values included.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
FLAGS = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined,float-cast-overflow",
         "-fno-sanitize-recover=all"]


def _build_and_run(cmd, exe):
    os.makedirs(OUT, exist_ok=True)
    r = subprocess.run(cmd + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert p.returncode == 0, p.stdout + p.stderr
    return p.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_abi_validation_under_sanitizers():
    exe = os.path.join(OUT, "abi_validation")
    cmd = ["g++", "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(ROOT, "block_quantized_amd", "csrc", "qmm.cpp"),
           os.path.join(SAN, "abi_stubs.cpp"), os.path.join(SAN, "abi_driver.cpp")]
    assert "abi validation ok" in _build_and_run(cmd, exe)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers():
    exe = os.path.join(OUT, "oracle_check")
    cmd = ["gcc", "-std=c11", *FLAGS, "-ffp-contract=off",
           os.path.join(ROOT, "oracle", "qmm_oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm"]
    assert "oracle ok" in _build_and_run(cmd, exe)
