"""The oracle and the library's host layer under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

``tests/sanitize/oracle_driver.c`` runs the fp64 oracle on small paged caches of
each kind (plain and split forms, several threads); ``tests/sanitize/host_driver.cpp``
runs the C ABI's host layer (``mla_api.cpp``) over a grid of shapes, page sizes and
cache types with the kernel launchers replaced by stubs that check the workspace
layout they are handed.  Both are built with gcc / g++ (host code only) and must
exit 0 with no sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _build_and_run(cmd, exe, tmp_path):
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    out = _build_and_run(["gcc", "-std=c11", *SAN, "-pthread", "tests/sanitize/oracle_driver.c",
                          "oracle/mla_oracle.c", "-o", str(exe), "-lm"], exe, tmp_path)
    assert "oracle driver ok" in out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not available")
def test_host_layer_under_sanitizers(tmp_path):
    exe = tmp_path / "host_driver"
    out = _build_and_run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-Iinclude",
                          "-Imla_attention_paged_amd/csrc", "tests/sanitize/host_driver.cpp",
                          "mla_attention_paged_amd/csrc/mla_api.cpp", "-o", str(exe)], exe, tmp_path)
    assert "host driver ok" in out
