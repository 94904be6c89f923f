"""The host-side plan code under sanitizers (no GPU).

tests/native/host_checks.cpp drives every host entry point of include/sta.h
(plan creation on fixed and seeded random shapes, every query, the error
paths, allocation failure injected at each allocation of a plan build, the
STA_TEST_FAIL_ALLOC hook) compiled with sta_plan.cpp under AddressSanitizer
+ UndefinedBehaviorSanitizer (LeakSanitizer on at exit), and, in a second
build, threads that take plans from the process-wide cache while another
thread keeps clearing it, under ThreadSanitizer.  Any sanitizer report fails
the test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sliding_tile_attention_sta_amd", "csrc")
SOURCES = [os.path.join(CSRC, "sta_plan.cpp"), os.path.join(ROOT, "tests", "native", "host_checks.cpp")]
INCLUDES = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
CXX = os.environ.get("CXX", "g++")

pytestmark = pytest.mark.skipif(shutil.which(CXX) is None, reason=f"{CXX} not found")


def build_and_run(tmp_path, name, flags, env_extra):
    exe = str(tmp_path / name)
    b = subprocess.run([CXX, "-std=c++17", "-O1", "-g", *flags, *INCLUDES, *SOURCES, "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-3000:]
    env = dict(os.environ, **env_extra)
    env.pop("STA_TEST_FAIL_ALLOC", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    return r


def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    r = build_and_run(tmp_path, "host_asan", ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
                      {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0", "UBSAN_OPTIONS": "print_stacktrace=1"})
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "LeakSanitizer" not in out and "runtime error" not in out
    assert ", 0 failed" in r.stdout
    n = int(r.stdout.split("host checks: ")[1].split(" checks")[0])
    assert n > 2000


def test_plan_cache_under_thread_sanitizer(tmp_path):
    r = build_and_run(tmp_path, "host_tsan", ["-fsanitize=thread", "-DHOST_CHECKS_THREADS"],
                      {"TSAN_OPTIONS": "halt_on_error=1"})
    out = r.stdout + r.stderr
    if "unexpected memory mapping" in out:
        pytest.skip("ThreadSanitizer cannot run under this kernel's address layout")
    assert r.returncode == 0, out[-4000:]
    assert "ThreadSanitizer" not in out
    assert "1 checks, 0 failed" in r.stdout
