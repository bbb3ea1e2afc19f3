"""Builds libasp.so (all HIP kernels + the C ABI) for gfx950 with hipcc.

Each translation unit is compiled to an object in parallel, then linked into
query_aware_sparse_amd/libasp.so (in-tree, next to this file).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libasp.so")
SOURCES = ["api.hip", "predict.hip", "score.hip", "select.hip", "attend.hip", "overlap.hip", "page.hip",
           "check.hip"]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build_library() -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    return LIB


C_ABI_DIR = os.path.join(ROOT, "tests", "c_abi")
C_ABI_CHECKS = ["step_check", "page_check"]


def build_c_abi_check() -> list:
    """The C++ programs that drive the C ABI without Python (tests/c_abi); they
    find libasp.so through a path relative to themselves."""
    built = []
    for name in C_ABI_CHECKS:
        out = os.path.join(C_ABI_DIR, name)
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=" + ARCH, "-O2", "-std=c++17", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I" + os.path.join(ROOT, "include"), os.path.join(C_ABI_DIR, name + ".cpp"), "-L" + PKG, "-lasp",
               "-Wl,-rpath,$ORIGIN/../../query_aware_sparse_amd", "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for the C ABI check:\n%s\n%s" % (" ".join(cmd), r.stderr))
        os.replace(tmp, out)
        built.append(out)
    return built


BENCH_DRIVER = os.path.join(ROOT, "bench_driver")


def build_bench_driver() -> str:
    """bench_driver.so, the C++ timing loop bench.py calls through ctypes; it
    finds libasp.so through a path relative to itself."""
    out = BENCH_DRIVER + ".so"
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-O2", "-std=c++17", "-Wall", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I" + os.path.join(ROOT, "include"), BENCH_DRIVER + ".cpp", "-L" + PKG, "-lasp",
           "-Wl,-rpath,$ORIGIN/query_aware_sparse_amd", "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for the bench driver:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library())
    print(build_c_abi_check())
    print(build_bench_driver())
