"""The C ABI's host code (ssd_api.cpp and ssd_bwd.cpp: validation, workspace
layout, launch plans, stage order) built with AddressSanitizer + UndefinedBehaviorSanitizer
and, separately, with ThreadSanitizer, against stub launchers that enqueue
nothing (tests/host/stub_launch.cpp), and driven through every validation
path and from eight threads at once (tests/host/abi_driver.cpp).  Plain g++,
host code only: no kernel is built or run."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "mamba_chunked_ssd_amd", "csrc", "ssd_api.cpp"),
           os.path.join(ROOT, "mamba_chunked_ssd_amd", "csrc", "ssd_bwd.cpp"),
           os.path.join(ROOT, "tests", "host", "stub_launch.cpp"),
           os.path.join(ROOT, "tests", "host", "abi_driver.cpp")]
ROCM_INCLUDE = "/opt/rocm/include"

needs_gxx = pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                               reason="needs g++ and the ROCm headers")


def _build_and_run(tmp_path, sanitize, env_extra):
    exe = str(tmp_path / ("abi_driver_" + sanitize.replace(",", "_")))
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I" + ROCM_INCLUDE, "-Wno-attributes", "-fsanitize=" + sanitize,
           "-fno-sanitize-recover=all", "-pthread"] + SOURCES + ["-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ)
    env.update(env_extra)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout[-2000:], r.stderr[-4000:])


@needs_gxx
def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    _build_and_run(tmp_path, "address,undefined",
                   {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
                    "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})


@needs_gxx
def test_host_code_under_thread_sanitizer(tmp_path):
    _build_and_run(tmp_path, "thread", {"TSAN_OPTIONS": "halt_on_error=1"})
