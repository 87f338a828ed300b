"""The host planner and page pool (plan.cpp, pool.cpp) under AddressSanitizer
and UndefinedBehaviorSanitizer: a C++ driver (tests/native/host_check.cpp)
runs the C ABI over random batches in every mode, re-plans, queue images,
error paths and a page-pool serving loop; a second driver
(tests/native/oom_check.cpp) makes allocations fail. Built with g++ (no HIP
kernels, no GPU); skipped where g++ or the sanitizer runtimes are missing."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_gqa_04_amd", "csrc")


def test_planner_and_pool_under_asan_and_ubsan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not found")
    exe = tmp_path / "host_check"
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "native", "host_check.cpp"),
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "pool.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr and "cannot find" in build.stderr:
        pytest.skip("sanitizer runtime not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe), "200"], capture_output=True, text=True, env=env, timeout=300)
    if run.returncode != 0 and "LeakSanitizer does not work under ptrace" in run.stderr:
        env["ASAN_OPTIONS"] = "detect_leaks=0"
        run = subprocess.run([str(exe), "200"], capture_output=True, text=True, env=env,
                             timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "host checks passed" in run.stdout
    assert "runtime error" not in run.stderr


def test_allocation_failures_return_a_status(tmp_path):
    # tests/native/oom_check.cpp replaces operator new with one that fails
    # once at a chosen allocation and walks that point over every
    # allocation of plan creation, re-planning and pool creation: each call
    # must return a status (an exception escaping the C ABI would end the
    # program), and a plan must re-plan normally afterwards.
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not found")
    exe = tmp_path / "oom_check"
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "native", "oom_check.cpp"),
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "pool.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "allocation failures handled" in run.stdout
