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
    out = bench.cpu_baseline(w, 4096 + 5, reps=1)
    assert out["kind"] == "oracle" and out["unit"] == "GB/s"
    one, mc = out["variants"]["oracle-1c"], out["variants"]["oracle-mc"]
    assert one["cores"] == 1 and mc["cores"] == min(len(os.sched_getaffinity(0)), w.nchannels)
    assert out["cores"] == mc["cores"] and out["value"] == mc["busbw_GBps"] > 0
    assert one["hbm_equiv_GBps"] > 0 and len(one["runs_s"]) == 1
    assert "4101 f32 elements per rank" in out["sample"]
    for key in ("cpu_model", "cores_available", "numpy", "python"):
        assert key in out["host"]


def test_multicore_oracle_step_computes_the_same_result():
    # The channels spread over threads write the same outputs as the plain
    # oracle (the channels' element ranges are disjoint).
    import numpy as np
    sys.path.insert(0, ROOT)
    from double_binary_tree_amd import inputs as I
    from oracle import allreduce as A
    from oracle import topology as T
    from concurrent.futures import ThreadPoolExecutor
    w = I.WORKLOADS["hier4x8_f16"]
    xs = I.rank_inputs(w, count=70001)
    for algo in ("ring", "tree"):
        want = A.allreduce(xs, w.nnodes, algo, w.nchannels, 4096, w.dtype, w.op)
        outs = [np.array(x, copy=True) for x in xs]
        topo = T.build_topology(w.nranks, w.nnodes, w.nchannels)
        with ThreadPoolExecutor(max_workers=4) as pool:
            list(pool.map(lambda c: A.allreduce_channel(xs, outs, c, topo, algo, 4096, w.dtype, w.op),
                          range(w.nchannels)))
        for a, b in zip(outs, want):
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
