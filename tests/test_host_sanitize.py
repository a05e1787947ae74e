"""The library's host helpers (routed_lora_delta_amd/csrc/rld_host.cpp: scale,
F16 -> BF16, rank padding, table packs, window and grid helpers) built with
g++ under AddressSanitizer and UndefinedBehaviorSanitizer together with
tests/host_sanitize_driver.cpp, which calls each of them at its edges on
exact-size heap buffers.  CPU only; skipped where g++ or the HIP headers are
missing."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP_INC = "/opt/rocm/include"


def test_host_helpers_clean_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(HIP_INC, "hip", "hip_runtime_api.h")):
        pytest.skip("g++ or the HIP headers are not available")
    exe = str(tmp_path / "host_sanitize")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INC,
           "-I", os.path.join(ROOT, "include"), "-include", "hip/hip_runtime_api.h",
           os.path.join(ROOT, "routed_lora_delta_amd", "csrc", "rld_host.cpp"),
           os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert run.stdout.strip().splitlines()[-1] == "ok"
