"""libopt8's host code under AddressSanitizer, UBSan and LeakSanitizer, on the CPU.

opt8_host.cpp (codebook and LUT construction, validation, the descriptor
cache, the scalar prologue, launch planning) is compiled with g++ together
with a host-only stand-in for the HIP runtime calls and the three kernel-side
functions it uses (tests/host_sanitize/fake_hip.cpp), and driven through every
entry point by tests/host_sanitize/driver.cpp.  No GPU code is built here.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CSRC = os.path.join(ROOT, "precision_optimizer_step_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


def _build(tmp_path, name, sanitizers, driver):
    if shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("g++ or the ROCm headers are missing")
    exe = tmp_path / name
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=" + sanitizers, "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I" + ROCM_INCLUDE, "-I" + os.path.join(ROOT, "include"),
           "-I" + CSRC, "-I" + HERE,
           os.path.join(CSRC, "opt8_host.cpp"), os.path.join(CSRC, "opt8_tables.cpp"), os.path.join(HERE, "fake_hip.cpp"),
           os.path.join(HERE, driver), "-pthread", "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "san" in build.stderr.lower() and "cannot find" in build.stderr.lower():
        pytest.skip("sanitizer runtime not installed")
    assert build.returncode == 0, build.stderr[-4000:]
    return exe


def test_host_code_is_clean_under_sanitizers(tmp_path):
    exe = _build(tmp_path, "opt8_host_driver", "address,undefined", "driver.cpp")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, (run.stdout[-4000:], run.stderr[-4000:])
    assert "all host checks passed" in run.stdout, run.stdout


def test_concurrent_callers_are_clean_under_thread_sanitizer(tmp_path):
    """Four threads step at once (shared and own lists, cache misses and evictions, every
    entry point); ThreadSanitizer must report no data race in the library's host code."""
    exe = _build(tmp_path, "opt8_host_threads", "thread", "threads.cpp")
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1:second_deadlock_stack=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert "ThreadSanitizer" not in run.stderr, run.stderr[-6000:]
    assert run.returncode == 0, (run.stdout[-4000:], run.stderr[-4000:])
    assert "all thread checks passed" in run.stdout, run.stdout
