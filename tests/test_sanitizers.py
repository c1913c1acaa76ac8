"""Host builds under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs are compiled with -fsanitize=address,undefined (every finding fatal) and run:
  * tests/c/oracle_host_check.c together with oracle/oracle.c: every oracle function on small
    inputs and its edge cases (empty sets, rows with no visible key, windows, grouped heads);
  * tests/c/api_host_check.cpp together with the C ABI layer
    exact_io_aware_31_amd/csrc/fa_api.cpp (host C++ only, with stand-in launchers that record
    their arguments): every validation path and the forwarding of valid calls.
Only host code is built here; no GPU code is compiled with a sanitizer.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")


def _need(tool):
    path = shutil.which(tool)
    if path is None:
        pytest.skip(f"{tool} not available")
    return path


def _build(cmd, tmp_path):
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp_path)
    if r.returncode != 0 and ("libasan" in r.stderr or "libubsan" in r.stderr):
        pytest.skip("sanitizer runtimes not installed: " + r.stderr[-300:])
    assert r.returncode == 0, r.stdout + r.stderr


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "0 failure(s)" in r.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return r.stdout


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    gcc = _need("gcc")
    exe = str(tmp_path / "oracle_host_check")
    _build([gcc, "-std=c11", "-Wall", "-Wextra", "-fopenmp", *SAN,
            os.path.join(ROOT, "tests", "c", "oracle_host_check.c"),
            os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", exe], tmp_path)
    out = _run(exe)
    assert out.count("ok  ") >= 20


def test_abi_layer_under_address_and_undefined_sanitizers(tmp_path):
    gxx = _need("g++")
    rocm_inc = "/opt/rocm/include"
    if not os.path.exists(os.path.join(rocm_inc, "hip", "hip_runtime.h")):
        pytest.skip("HIP headers not available")
    exe = str(tmp_path / "api_host_check")
    csrc = os.path.join(ROOT, "exact_io_aware_31_amd", "csrc")
    _build([gxx, "-std=c++17", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I", rocm_inc,
            "-I", os.path.join(ROOT, "include"), "-I", csrc, *SAN,
            os.path.join(ROOT, "tests", "c", "api_host_check.cpp"),
            os.path.join(csrc, "fa_api.cpp"), "-o", exe], tmp_path)
    out = _run(exe)
    assert out.count("ok  ") >= 30
