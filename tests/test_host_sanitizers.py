"""The library's host code (host_api.cpp: page pool, block tables, byte
accounting, split plan) built with g++ under AddressSanitizer, its leak
checker and UndefinedBehaviorSanitizer, driven by tests/sanitize/host_driver.cpp
(error paths and a seeded random reserve / fork / copy-on-write / release
schedule checked against a shadow model).  Host code only: nothing here runs
on a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_254_amd", "csrc")
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")


def _build(tmp_path, sanitizers):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = tmp_path / "host_driver"
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-Wall", "-Wextra", "-fno-omit-frame-pointer",
           f"-fsanitize={sanitizers}", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", ROCM_INCLUDE,
           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"), os.path.join(CSRC, "host_api.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


def test_host_code_under_sanitizers(tmp_path):
    exe = _build(tmp_path, "address,undefined")
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "host driver: ok" in r.stdout
    assert "runtime error" not in r.stderr      # UBSan reports, even if recovered
