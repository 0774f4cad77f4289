"""bench.py's contract on a machine without a GPU: more than one GPU is
refused with a message, a missing GPU is an error rather than a CPU run,
and the host-side oracle baseline reports what the JSON line needs."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    p = _run("--gpus", "2")
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_no_gpu_is_an_error_not_a_cpu_run():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    p = _run("--steps", "1", "--warmup", "0")
    assert p.returncode == 2
    assert "needs a GPU" in p.stderr
    assert p.stdout == ""


def test_cpu_baseline_fields():
    sys.path.insert(0, ROOT)
    import bench
    from double_binary_tree_amd import inputs as I
    w = I.WORKLOADS[bench.WORKLOAD]
    out = bench.cpu_baseline(w, 4096 + 5, 0.0)
    assert out["kind"] == "oracle" and out["unit"] == "GB/s" and out["cores"] == 1
    assert out["value"] > 0
    assert "4101 f32 elements per rank" in out["sample"]
