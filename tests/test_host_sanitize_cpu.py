"""The library's host-only code (pop_host.cpp: status strings, the last-error
buffer, region counts, top-k counts and the index-list check) built with g++
under AddressSanitizer and UndefinedBehaviorSanitizer, and driven through its
argument range by tests/host_sanitize_driver.cpp, which self-checks every
result.  Any out-of-bounds access, overflow or other undefined behaviour ends
the run with a sanitizer report.  CPU only: no device code is built."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is not installed")
def test_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_sanitize")
    build = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
             "-o", exe, os.path.join(HERE, "host_sanitize_driver.cpp"),
             os.path.join(ROOT, "online_structured_ffn_amd", "csrc", "pop_host.cpp")]
    r = subprocess.run(build, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0:detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout
    assert int(r.stdout.split()[1]) > 100000
