"""The host half of libprkv.so under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/host_sanitize_driver.cpp drives
descriptor validation, the fact table, build_slot_mapping and
rope_table_fill with seeded random valid and invalid inputs; the driver and
prkv_host.cpp are built with g++ (host code only, no device code)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_library_under_asan_ubsan(tmp_path):
    exe = tmp_path / "host_sanitize"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "pre_rope_kv_amd", "csrc"),
           os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"),
           os.path.join(ROOT, "pre_rope_kv_amd", "csrc", "prkv_host.cpp"), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "0 failures" in run.stdout
