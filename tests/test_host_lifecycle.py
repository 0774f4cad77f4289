"""Resource handling of the library's host code (CPU only).

tests/host/lifecycle_check.cpp drives the C ABI of api.cpp, built with g++
under AddressSanitizer and UndefinedBehaviorSanitizer against a host-only
stand-in for the HIP runtime and the kernel launchers
(tests/host/fake_hip.cpp), which tracks every device allocation and checks
every table pointer a launch receives.  It checks that emu_comm_destroy
frees every device allocation (tables, FIFO workspaces, LL status words),
that dropping cached communicators frees theirs, that
emu_allreduce_noalloc never allocates and hands its kernels the same tables
as emu_allreduce (across shape changes), and what it refuses."""

import os
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "double_binary_tree_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")
BUILD = os.path.join(ROOT, "_build", "host_tests")


def test_lifecycle_under_sanitizers():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "lifecycle_check")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include", "-I" + CSRC, "-I" + os.path.join(ROOT, "include"),
           "-I" + HOST, os.path.join(HOST, "lifecycle_check.cpp"), os.path.join(HOST, "fake_hip.cpp"),
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "topology.cpp"),
           "-o", exe + f".{os.getpid()}"]
    subprocess.run(cmd, check=True, capture_output=True)
    os.replace(exe + f".{os.getpid()}", exe)   # atomic: parallel workers may run the previous build
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1")
    env.pop("EMU_DEBUG", None)
    out = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stderr[-4000:]
