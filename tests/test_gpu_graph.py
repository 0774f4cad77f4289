"""Parity of per-channel rank orders and the split / balanced head patterns
(HIP path through the C ABI against the oracle), bit-exact.

Cases: the per-channel chains of the pages' 4-GPU table ("NCCL 专家课程 13",
section "从 GRAPH 日志复原 active tree"), seeded random per-channel orders
(several distinct orders per communicator, so the fused kernel reads its
order table and the stepwise ring maps positions to ranks), and the three
head patterns on hierarchical shapes."""

from dataclasses import replace

import numpy as np
import pytest

from double_binary_tree_amd import inputs as I
from oracle import allreduce as A
from tests.gpu_util import announce, check_every_element, clear_inputs, run_allreduce

pytestmark = pytest.mark.gpu

TABLE4 = [[0, 1, 2, 3], [0, 1, 2, 3], [0, 2, 1, 3], [0, 2, 1, 3], [1, 0, 3, 2], [1, 0, 3, 2],
          [0, 1, 2, 3], [0, 1, 2, 3], [0, 2, 1, 3], [0, 2, 1, 3], [1, 0, 3, 2], [1, 0, 3, 2]]

_hier = I.WORKLOADS["hier4x8_f16"]
_chain = I.WORKLOADS["chain8_f32"]
# name -> (workload shape, pattern, per-channel orders)
GRAPHS = {
    "table4_f32": (replace(_chain, name="table4_f32", nranks=4, nchannels=12), "tree", TABLE4),
    "table4_bf16": (replace(_chain, name="table4_bf16", nranks=4, nchannels=12, dtype="bf16"), "tree", TABLE4),
    "orders8_f32": (replace(_chain, name="orders8_f32", nchannels=6), "tree", I.intra_orders(8, 1, 6, 101)),
    "split4x8_f16": (_hier, "split", I.intra_orders(32, 4, 16, 102)),
    "balanced4x8_f16": (_hier, "balanced", I.intra_orders(32, 4, 16, 103)),
    "split4x8_i64": (I.WORKLOADS["hier4x8_i64"], "split", None),
    "balanced4x8_f32max": (I.WORKLOADS["hier4x8_f32max"], "balanced", I.intra_orders(32, 4, 16, 104)),
    "split3x2_f32": (replace(_chain, name="split3x2_f32", nranks=6, nnodes=3, nchannels=4), "split",
                     I.intra_orders(6, 3, 4, 105)),
    "balanced8x2_bf16": (replace(_hier, name="balanced8x2_bf16", nranks=16, nnodes=8, nchannels=6, dtype="bf16"),
                         "balanced", I.intra_orders(16, 8, 6, 106)),
    "split32x2_f32": (replace(_chain, name="split32x2_f32", nranks=64, nnodes=32, nchannels=8), "split",
                      I.intra_orders(64, 32, 8, 107)),
}
RTOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from double_binary_tree_amd import emucomm as E
    E.lib()
    yield
    clear_inputs()
    E.comm_destroy()
    torch.cuda.empty_cache()


def _bits(x):
    return np.ascontiguousarray(x).view(np.uint8)


def _check(name, algo, mode, count, chunk_bytes, inplace, salt=0):
    w, pattern, intra = GRAPHS[name]
    announce(f"graph {name} pattern={pattern} algo={algo} mode={mode} count={count} chunk={chunk_bytes} "
             f"inplace={inplace}")
    xs = I.rank_inputs(w, count=count, salt=salt)
    want = A.allreduce(xs, w.nnodes, algo, w.nchannels, chunk_bytes, w.dtype, w.op, pattern=pattern, intra=intra)[0]
    got, _ = run_allreduce(xs, w.nnodes, algo, mode, w.nchannels, chunk_bytes, w.dtype, w.op, inplace,
                           pattern=pattern, intra=intra)
    wb = _bits(want).reshape(len(want), -1)
    for r, g in enumerate(got):
        gb = _bits(g).reshape(len(g), -1)
        if not np.array_equal(gb, wb):
            bad = np.nonzero((gb != wb).any(axis=1))[0]
            raise AssertionError(f"rank {r}: {len(bad)} elements differ, first at {bad[:8].tolist()}")
    if w.dtype in RTOL and w.op == "sum":
        ok, err = A.within_tolerance(got[0], xs, w.dtype, RTOL[w.dtype])
        assert ok, err


CASES = [(name, algo, mode) for name in GRAPHS for algo in ("ring", "tree") for mode in ("fused", "stepwise")]


@pytest.mark.parametrize("name,algo,mode", CASES)
@pytest.mark.parametrize("inplace", [False, True])
def test_graph_parity_small_chunks(name, algo, mode, inplace):
    w = GRAPHS[name][0]
    unit = 16 // w.itemsize
    count = 37 * 1024 + 3 * unit + (1 if unit > 1 else 0)
    _check(name, algo, mode, count, chunk_bytes=4096, inplace=inplace)


@pytest.mark.parametrize("name", ["table4_f32", "split4x8_f16", "orders8_f32"])
@pytest.mark.parametrize("algo", ["ring", "tree"])
@pytest.mark.parametrize("mode", ["fused", "stepwise"])
def test_graph_parity_edge_counts(name, algo, mode):
    for count in (1, 2, 3, 7, 8, 9, 17, 257, 1025, 4099):
        _check(name, algo, mode, count, chunk_bytes=64, inplace=False, salt=2)


@pytest.mark.parametrize("algo", ["ring", "tree"])
@pytest.mark.parametrize("name", ["split4x8_f16", "orders8_f32", "table4_bf16", "balanced4x8_f32max"])
def test_graph_full_size_every_element(name, algo):
    # The workload's full size and chunk with the graph's pattern and
    # per-channel orders: every element of every rank equals the oracle's,
    # fused and stepwise, out of place and in place.
    w, pattern, intra = GRAPHS[name]
    check_every_element(w, algo, pattern=pattern, intra=intra, label=f"graph {name} ")
