"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the host code (CPU only).

* kda_abi.cpp -- the C ABI's argument checks, workspace layout and launch sequencing --
  built with the host compiler against stand-in launchers (tests/sanitize/abi_stubs.cpp)
  and driven through every status code (tests/sanitize/abi_driver.cpp);
* the float64 oracle (oracle/kda_oracle.c) on a small packed batch with an empty
  sequence, every gate form and the chunk-start states (tests/sanitize/oracle_driver.c).

Each build runs once; any sanitizer report fails the test.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"), reason="needs g++ and HIP headers")
def test_abi_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_asan")
    rc, out = _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I" + os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "gated_delta_rule_log2_amd", "csrc", "kda_abi.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "abi_stubs.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"),
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe], str(tmp_path))
    assert rc == 0, out
    rc, out = _run([exe], str(tmp_path))
    assert rc == 0 and "abi driver ok" in out and "runtime error" not in out and "ERROR:" not in out, out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    rc, out = _run(["gcc", "-std=c11", *SAN, "-pthread", os.path.join(ROOT, "oracle", "kda_oracle.c"),
                    os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm", "-o", exe], str(tmp_path))
    assert rc == 0, out
    rc, out = _run([exe], str(tmp_path))
    assert rc == 0 and "oracle driver ok" in out and "runtime error" not in out and "ERROR:" not in out, out
