"""Build libemucomm.so in-tree: HIP kernels for gfx950 with hipcc, host C++
with g++, linked by hipcc.  ``python -m double_binary_tree_amd.build``."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libemucomm.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIP_SOURCES = ["fused.hip", "stepwise.hip", "ll.hip", "xwg.hip", "noalloc.hip", "stream.hip"]
CXX_SOURCES = ["api.cpp", "plan.cpp", "topology.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # No packed-FP32 instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Keep subnormals and never contract: the reductions must round exactly
    # as the element type's own add does.
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-Wextra", "-Wno-unused-parameter",
             f"-I{ROCM}/include", "-D__HIP_PLATFORM_AMD__"]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in proc.stdout.splitlines()
                    if "packed-fp32-ops" not in ln and "not a recognized feature" not in ln)
    if proc.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{proc.stdout}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    cxx = shutil.which("g++") or "g++"
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([cxx, *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as pool:
        for out in pool.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs,
          f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"])
    os.replace(tmp, LIB)
    return LIB


def build_capi_check() -> str:
    """The C program that exercises the ABI from plain C (tests/host/capi_check.c),
    built as a shared library that the GPU tests load in-process; it links
    libemucomm.so from the package directory."""
    src = os.path.join(ROOT, "tests", "host", "capi_check.c")
    out = os.path.join(ROOT, "tests", "host", "libcapi_check.so")
    cc = shutil.which("gcc") or "gcc"
    tmp = out + ".tmp"
    _run([cc, "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
          f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", src, "-o", tmp,
          f"-L{PKG}", "-lemucomm", "-Wl,-rpath,$ORIGIN/../../double_binary_tree_amd", f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{ROCM}/lib"])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
