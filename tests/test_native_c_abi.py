"""The C ABI from plain C (CPU only): tests/native/c_abi_smoke.c includes
include/pf.h, is compiled as strict C99 with every warning an error, links
the built libpf.so and runs host-only allocator calls with their documented
results and error codes."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "paged_kv_cache_43_amd")


def test_header_and_library_from_c99(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(LIB_DIR, "libpf.so")):
        pytest.fail("libpf.so is not built (run __graft_entry__.build())")
    exe = str(tmp_path / "c_abi_smoke")
    cmd = ["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "native", "c_abi_smoke.c"), "-L", LIB_DIR, "-lpf",
           "-Wl,-rpath," + LIB_DIR, "-o", exe]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert r.returncode == 0 and "c abi ok" in r.stdout, r.stdout[-3000:]
