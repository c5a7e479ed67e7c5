"""Build libpf.so in-tree: the host allocator with g++, the HIP kernels with
hipcc for gfx950, linked into ``paged_kv_cache_43_amd/libpf.so``.

Run ``python -m paged_kv_cache_43_amd.build`` (or ``__graft_entry__.build()``).
Every HIP file is compiled with packed-fp32 instructions disabled.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpf.so")
ARCH = "gfx950"

HIP_SOURCES = ["pf_kv.hip", "pf_attn.hip", "pf_attn_mfma.hip"]
HOST_SOURCES = ["pf_host.cpp"]


def _hipcc():
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def hip_flags():
    return ["-O3", "-std=c++17", "--offload-arch=" + ARCH, "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build step failed: %s\n%s" % (" ".join(cmd), out))
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-c",
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([hipcc] + hip_flags() + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
