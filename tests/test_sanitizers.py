"""CPU sanitizer leg: the host side of the C ABI and the CPU oracle built with
AddressSanitizer and UndefinedBehaviorSanitizer (gcc / g++ only; nothing here is built
for the GPU) and run clean.

* cv_api.cpp - every entry point's validation and launch planning - is linked with
  tests/c/hip_host_stub.cpp in place of the device code and the HIP runtime: the stub's
  kernel pickers return markers and its hipLaunchKernel records the launch instead of
  running it.  tests/c/abi_sanitize.cpp checks the kernel, grid and launch choices of
  the benchmark shapes, the refusals (code, detail, nothing launched), a launch failure,
  and a fuzz of a million random shapes over the full range of every field: a refused
  call launches nothing, an accepted one launches one grid within the hardware limits.
* oracle/conv_verify_oracle.c runs every kind of problem from tests/c/oracle_sanitize.c
  with each buffer a heap block of exactly its size, plus the refusals.

Any sanitizer report aborts the program (-fno-sanitize-recover=all), and leaks are
reported at exit.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C_DIR = os.path.join(ROOT, "tests", "c")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1", HIP_VISIBLE_DEVICES="-1")


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not found")


def _build_and_run(cmd, exe, args=()):
    cc = subprocess.run(cmd, capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([exe, *args], capture_output=True, text=True, env=ENV, timeout=300)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "MISMATCH" not in out and "runtime error" not in out and "ERROR: " not in out, out[-4000:]
    assert out.rstrip().endswith("ALL OK"), out[-2000:]
    return out


def test_abi_host_code_under_asan_ubsan(tmp_path):
    _need("g++")
    hip_inc = "/opt/rocm/include"
    if not os.path.exists(os.path.join(hip_inc, "hip", "hip_runtime_api.h")):
        pytest.skip("HIP headers not found")
    exe = str(tmp_path / "abi_sanitize")
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", f"-I{hip_inc}",
           f"-I{os.path.join(ROOT, 'include')}",
           f"-I{os.path.join(ROOT, 'causal_conv1d_verify_amd', 'csrc')}",
           os.path.join(ROOT, "causal_conv1d_verify_amd", "csrc", "cv_api.cpp"),
           os.path.join(C_DIR, "hip_host_stub.cpp"), os.path.join(C_DIR, "abi_sanitize.cpp"),
           "-o", exe]
    out = _build_and_run(cmd, exe, ["1000000"])
    assert "fuzz: 1000000 shapes" in out


def test_oracle_under_asan_ubsan(tmp_path):
    _need("gcc")
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", *SAN, os.path.join(ROOT, "oracle", "conv_verify_oracle.c"),
           os.path.join(C_DIR, "oracle_sanitize.c"), "-lm", "-o", exe]
    _build_and_run(cmd, exe)
