"""EMU_ALGO_AUTO on the GPU: each all-reduce runs the algorithm the cost
model selects for its size, and its bits are the oracle's for that
algorithm."""

import numpy as np
import pytest

from double_binary_tree_amd import inputs as I
from oracle import allreduce as A
from oracle import costmodel as CM
from oracle import topology as T
from tests.gpu_util import announce, run_allreduce

pytestmark = pytest.mark.gpu

CLASS_RANKS = (8, 16, 32)       # one rank count inside each rank-count class of the cost model
DEFAULTS = {}


def _restore():
    from double_binary_tree_amd import emucomm as E
    for (mode, algo, n), (a, b) in DEFAULTS.items():
        E.set_cost_model_ranks(algo, mode, n, a, b)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from double_binary_tree_amd import emucomm as E
    E.lib()
    for mode in ("stepwise", "fused"):
        for algo in ("ring", "tree"):
            for n in CLASS_RANKS:
                DEFAULTS[(mode, algo, n)] = E.get_cost_model(algo, mode, n)
    yield
    _restore()
    E.comm_destroy()


@pytest.mark.parametrize("name", ["chain8_f32", "dtree16_bf16", "hier4x8_f16"])
@pytest.mark.parametrize("mode", ["fused", "stepwise"])
def test_auto_runs_the_selected_algorithm(name, mode):
    from double_binary_tree_amd import emucomm as E
    w = I.WORKLOADS[name]
    depth = max(ch.true_depth() for ch in T.build_topology(w.nranks, w.nnodes, w.nchannels).channels)
    # parameters whose crossover falls inside the tested sizes: the tree has
    # the cheaper stages, the ring the higher bandwidth
    ring, tree = (3.0, 2.0e6), (0.5, 1.0e4)
    E.set_cost_model("ring", mode, *ring)
    E.set_cost_model("tree", mode, *tree)
    try:
        seen = set()
        for count in (1000, 4099, 60000, 600001):
            s = float(count) * w.itemsize
            want_algo = CM.select(w.nranks, depth, s, ring + (0.0,), tree + (0.0,))
            E.comm_init(w.nranks, w.nnodes, "auto", w.nchannels, 4096, mode=mode)
            assert E.select_algo(count, w.dtype) == want_algo
            seen.add(want_algo)
            announce(f"auto {name} {mode} count={count} -> {want_algo}")
            xs = I.rank_inputs(w, count=count, salt=7)
            want = A.allreduce(xs, w.nnodes, want_algo, w.nchannels, 4096, w.dtype, w.op)[0]
            got, _ = run_allreduce(xs, w.nnodes, "auto", mode, w.nchannels, 4096, w.dtype, w.op)
            for g in got:
                assert np.array_equal(np.ascontiguousarray(g).view(np.uint8), np.ascontiguousarray(want).view(np.uint8))
        assert seen == {"ring", "tree"}
    finally:
        _restore()
