"""Parity of the HIP all-reduce (through the C ABI) with the CPU oracle.

Bar: bit-exact for every element type, since the kernels evaluate every
element in the oracle's own order (integers: exact; floats: order-matched
with per-hop rounding).  Float results are also held to the float64 bound.
"""

import numpy as np
import pytest

from double_binary_tree_amd import inputs as I
from oracle import allreduce as A
from tests.gpu_util import announce, run_allreduce

pytestmark = pytest.mark.gpu

RTOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from double_binary_tree_amd import emucomm as E
    E.lib()   # a missing library is an error on a GPU machine
    yield
    E.comm_destroy()


def _bits(x):
    return np.ascontiguousarray(x).view(np.uint8)


def _check(w, algo, mode, count, chunk_bytes, inplace, salt=0):
    announce(f"{w.name} algo={algo} mode={mode} count={count} chunk={chunk_bytes} inplace={inplace}")
    xs = I.rank_inputs(w, count=count, salt=salt)
    want = A.allreduce(xs, w.nnodes, algo, w.nchannels, chunk_bytes, w.dtype, w.op)[0]
    got, _ = run_allreduce(xs, w.nnodes, algo, mode, w.nchannels, chunk_bytes, w.dtype, w.op, inplace)
    wb = _bits(want).reshape(len(want), -1)
    for r, g in enumerate(got):
        gb = _bits(g).reshape(len(g), -1)
        if not np.array_equal(gb, wb):
            first = np.nonzero((gb != wb).any(axis=1))[0]
            raise AssertionError(f"rank {r}: {len(first)} elements differ, first at {first[:8].tolist()}"
                                 f" got {g[first[:4]]} want {want[first[:4]]}")
    if w.dtype in RTOL and w.op == "sum":
        ok, err = A.within_tolerance(got[0], xs, w.dtype, RTOL[w.dtype])
        assert ok, err


CASES = []
for name, w in I.WORKLOADS.items():
    for algo in w.algos:
        for mode in ("fused", "stepwise"):
            CASES.append((name, algo, mode))


@pytest.mark.parametrize("name,algo,mode", CASES)
@pytest.mark.parametrize("inplace", [False, True])
def test_parity_small_chunks(name, algo, mode, inplace):
    # Small chunks so that a modest count spans many chunks, ring loops,
    # tiles and workgroup tasks, with a ragged tail.
    w = I.WORKLOADS[name]
    unit = 16 // w.itemsize
    count = 37 * 1024 + 3 * unit + (1 if unit > 1 else 0)
    _check(w, algo, mode, count, chunk_bytes=4096, inplace=inplace)


@pytest.mark.parametrize("name,algo,mode", CASES)
def test_parity_workload_chunk(name, algo, mode):
    # The workload's own chunk size at a count the oracle finishes quickly.
    w = I.WORKLOADS[name]
    count = min(w.count, 300_000 + 5)
    _check(w, algo, mode, count, chunk_bytes=w.chunk_bytes, inplace=False, salt=1)


EDGE_COUNTS = [1, 2, 3, 7, 8, 9, 15, 16, 17, 255, 256, 257, 1023, 1024, 1025, 4099]


@pytest.mark.parametrize("mode", ["fused", "stepwise"])
@pytest.mark.parametrize("algo", ["ring", "tree"])
@pytest.mark.parametrize("dtype,op", [("f32", "sum"), ("bf16", "sum"), ("f16", "max"), ("i64", "sum")])
def test_edge_counts(algo, mode, dtype, op):
    base = I.Workload("edge", 7, 6, 3, (algo,), 5, 64, dtype, op, 1,
                      ("int", -50, 50) if dtype.startswith("i") else ("normal", 1.0))
    for count in EDGE_COUNTS:
        _check(base, algo, mode, count, chunk_bytes=64, inplace=(count % 2 == 1))


@pytest.mark.parametrize("mode", ["fused", "stepwise"])
@pytest.mark.parametrize("n,m,nch", [(1, 1, 1), (2, 1, 1), (2, 2, 3), (3, 3, 2), (5, 5, 7),
                                     (12, 3, 4), (17, 17, 2), (24, 4, 6), (33, 3, 3), (64, 8, 64),
                                     (64, 64, 2), (48, 2, 1)])
@pytest.mark.parametrize("algo", ["ring", "tree"])
def test_shapes(n, m, nch, algo, mode):
    w = I.Workload("shape", 8, n, m, (algo,), nch, 256, "f32", "sum", 1, ("normal", 1.0))
    _check(w, algo, mode, 6 * 1024 + 13, chunk_bytes=256, inplace=False)


@pytest.mark.parametrize("n", list(range(1, 41)))
@pytest.mark.parametrize("algo,per_node", [("ring", False), ("tree", False), ("tree", True)])
def test_fused_every_rank_count(n, algo, per_node):
    """The fused pass loads a lane's inputs in batches (8 up to 8 ranks,
    else 16) and folds the ranks past the last whole batch in one more
    phase: every rank count from 1 to 40 covers every remainder of both
    batches, for the ring and chain folds (one node) and for the
    register-stack programs of the double tree (one rank per node); ragged
    count, bf16 so that every hop rounds."""
    nodes = n if per_node else 1
    w = I.Workload("ranks", 8, n, nodes, (algo,), 3, 4096, "bf16", "sum", 1, ("normal", 1.0))
    _check(w, algo, "fused", 3 * 1024 + 11, chunk_bytes=4096, inplace=False, salt=n)


@pytest.mark.parametrize("n", list(range(1, 41)))
@pytest.mark.parametrize("algo,per_node", [("ring", False), ("tree", False), ("tree", True)])
def test_stepwise_every_rank_count(n, algo, per_node):
    """The stepwise kernels change form with the rank count: one rank per
    wave up to 16 ranks, two up to 32, four beyond; the ring's load queue
    runs past the last step below 4 ranks; a chain's depth and a double
    tree's shape change with every count.  Every count from 1 to 40, ragged
    count, bf16."""
    nodes = n if per_node else 1
    w = I.Workload("ranks", 8, n, nodes, (algo,), 3, 4096, "bf16", "sum", 1, ("normal", 1.0))
    _check(w, algo, "stepwise", 3 * 1024 + 11, chunk_bytes=4096, inplace=False, salt=n)


@pytest.mark.parametrize("mode", ["fused", "stepwise"])
def test_count_zero_is_noop(mode):
    import torch
    from double_binary_tree_amd import emucomm as E
    E.comm_init(4, 2, "tree", 2, 4096, mode=mode)
    sends = [torch.full((8,), float(r), device="cuda") for r in range(4)]
    recvs = [torch.full((8,), -1.0, device="cuda") for _ in range(4)]
    E.allreduce([s.data_ptr() for s in sends], [r.data_ptr() for r in recvs], 0, "f32", "sum",
                torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert all(bool((r == -1.0).all()) for r in recvs)


@pytest.mark.parametrize("algo,mode", [("ring", "fused"), ("tree", "fused"), ("ring", "stepwise"),
                                       ("tree", "stepwise")])
def test_deterministic_and_modes_agree(algo, mode):
    w = I.WORKLOADS["hier4x8_f16"] if algo == "tree" else I.WORKLOADS["chain8_f32"]
    xs = I.rank_inputs(w, count=200_003, salt=2)
    announce(f"determinism {w.name} {algo} {mode}")
    a, sends = run_allreduce(xs, w.nnodes, algo, mode, w.nchannels, w.chunk_bytes, w.dtype, w.op)
    b, _ = run_allreduce(xs, w.nnodes, algo, mode, w.nchannels, w.chunk_bytes, w.dtype, w.op, sends=sends)
    other = "stepwise" if mode == "fused" else "fused"
    c, _ = run_allreduce(xs, w.nnodes, algo, other, w.nchannels, w.chunk_bytes, w.dtype, w.op, sends=sends)
    for x, y, z in zip(a, b, c):
        assert np.array_equal(_bits(x), _bits(y))
        assert np.array_equal(_bits(x), _bits(z))


@pytest.mark.parametrize("name,mode", [("hier4x8_f16", "fused"), ("hier4x8_f16", "stepwise"),
                                       ("dtree16_bf16", "fused"), ("dtree16_bf16", "stepwise"),
                                       ("dtree16_bf16", "ll")])   # LL in LDS: at most 16 ranks
def test_parity_in_library_layout(name, mode):
    """Buffers placed by emu_buffer_layout (one pool, staggered slots):
    the same bits as the oracle."""
    import torch
    from double_binary_tree_amd import emucomm as E
    from tests.gpu_util import to_device, to_host_bits
    w = I.WORKLOADS[name]
    count = 200_003
    announce(f"library layout {name} {mode} count={count}")
    xs = I.rank_inputs(w, count=count, salt=3)
    algo = w.algos[0]
    want = A.allreduce(xs, w.nnodes, algo, w.nchannels, w.chunk_bytes, w.dtype, w.op)[0]
    tdt = to_device(xs[0][:1], w.dtype).dtype
    pool, sends, recvs = E.rank_buffers(w.nranks, count, tdt)
    for s_, x in zip(sends, xs):
        s_.copy_(to_device(x, w.dtype))
    E.comm_init(w.nranks, w.nnodes, algo, w.nchannels, w.chunk_bytes, mode=mode)
    E.allreduce_tensors(sends, recvs, w.op)
    torch.cuda.synchronize()
    for r in recvs:
        assert np.array_equal(_bits(to_host_bits(r, w.dtype)), _bits(want))
    if mode == "ll":
        assert not E.protocol_status()
    del pool, sends, recvs


@pytest.mark.parametrize("mode", ["fused", "stepwise", "ll"])
def test_two_streams_at_once(mode):
    """Calls of one communicator on two streams, enqueued back to back
    without a wait between them (the fused, stepwise and LL kernels keep no
    state on the device between calls: their tables are read-only), each on
    its own buffers: both results are the oracle's."""
    import torch
    from double_binary_tree_amd import emucomm as E
    from tests.gpu_util import to_device, to_host_bits
    w = I.Workload("streams", 9, 8, 2, ("tree",), 6, 8192, "f32", "sum", 1, ("normal", 1.0))
    count = 300_007
    E.comm_init(w.nranks, w.nnodes, "tree", w.nchannels, w.chunk_bytes, mode=mode)
    sets = []
    for salt in (21, 22):
        xs = I.rank_inputs(w, count=count, salt=salt)
        sends = [to_device(x, "f32") for x in xs]
        recvs = [torch.empty_like(s) for s in sends]
        sets.append((xs, sends, recvs))
    E.allreduce_tensors(sets[0][1], sets[0][2], "sum")   # builds the plan outside the concurrent part
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    for st, (_, sends, recvs) in zip(streams, sets):
        E.allreduce([s.data_ptr() for s in sends], [r.data_ptr() for r in recvs], count, "f32", "sum",
                    st.cuda_stream)
    torch.cuda.synchronize()
    if mode == "ll":
        assert not E.protocol_status()
    for xs, _, recvs in sets:
        want = A.allreduce(xs, w.nnodes, "tree", w.nchannels, w.chunk_bytes, "f32", "sum")[0]
        for r in recvs:
            assert np.array_equal(_bits(to_host_bits(r, "f32")), _bits(want))
