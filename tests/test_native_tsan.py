"""Thread safety of the host allocator under ThreadSanitizer (CPU only):
tests/native/tsan_stress.cpp is built with g++ -fsanitize=thread against
csrc/pf_host.cpp alone and run; any data race or unexpected status fails."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_allocator_under_thread_sanitizer(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "tsan_stress")
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fsanitize=thread", "-pthread",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "paged_kv_cache_43_amd", "csrc"),
           os.path.join(ROOT, "tests", "native", "tsan_stress.cpp"),
           os.path.join(ROOT, "paged_kv_cache_43_amd", "csrc", "pf_host.cpp"), "-o", exe]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0 and "tsan" in r.stdout.lower():
        pytest.skip("ThreadSanitizer runtime not available: " + r.stdout[-300:])
    assert r.returncode == 0, r.stdout
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=240)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "failures 0, pool whole 1" in r.stdout
