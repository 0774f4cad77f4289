"""Register budgets the planner relies on (CPU: compiles the stepwise
kernels for gfx950 and reads the compiler's resource report).

The stepwise plans size their grids from HIP's occupancy query, which does
not count scalar registers, while the hardware holds fewer waves per SIMD
once a wave's SGPR allocation passes 80 (measured on MI355X: 8 waves at 78
SGPRs, 7 at 86, 6 at 102).  The one-rank-per-wave kernels must therefore
stay within 80 SGPRs, or a quarter of the planned workgroups would wait for
a slot."""

import os
import re
import shutil
import subprocess

import pytest

from double_binary_tree_amd import build as B

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")


@pytest.fixture(scope="module")
def report(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("res") / "stepwise.o"
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-fPIC", "-Wall", "-Wno-unused-function")]
    proc = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-c", os.path.join(B.CSRC, "stepwise.hip"),
                           "-o", str(out), "-Rpass-analysis=kernel-resource-usage"],
                          stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert proc.returncode == 0, proc.stdout[-2000:]
    kernels = {}
    name = None
    for line in proc.stdout.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+(TotalSGPRs|VGPRs|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and name:
            kernels[name][m.group(1)] = int(m.group(2))
    return kernels


def _one_rank_per_wave(kernels, kind):
    # step_tree<Red, ESZ, RPW> and step_ring<Red, ESZ, COLL, RPW>: RPW = 1 ends the template list
    pat = re.compile(rf"^_ZN3emu9{kind}.*Li1EEEvNS_8StepArgs")
    return {k: v for k, v in kernels.items() if pat.search(k)}


@pytest.mark.parametrize("kind", ["step_tree", "step_ring"])
def test_one_rank_per_wave_kernels_fit_80_sgprs(report, kind):
    ks = _one_rank_per_wave(report, kind)
    assert len(ks) >= 10, f"found {len(ks)} {kind} instantiations with one rank per wave"
    over = {k: v["TotalSGPRs"] for k, v in ks.items() if v["TotalSGPRs"] > 80}
    assert not over, f"{kind} kernels above 80 SGPRs (fewer waves per SIMD than planned): {over}"
    low = {k: v["Occupancy [waves/SIMD]"] for k, v in ks.items() if v["Occupancy [waves/SIMD]"] < 8}
    assert not low, f"{kind} kernels below 8 waves per SIMD: {low}"
