"""Parity of the stepwise all-reduce under the LL protocol (EMU_PROTO_LL)
with the CPU oracle, through the C ABI.

The protocol changes how a step's data reaches the next rank (flag-in-line
FIFO words polled by the reader, consumed counts published back), never
the order of any reduction, so the bar is the same as for the slot
protocol: bit-exact to the oracle for every type.  Every case also checks
that no call was abandoned (emu_protocol_status)."""

import numpy as np
import pytest

from double_binary_tree_amd import inputs as I
from oracle import allreduce as A
from tests.gpu_util import announce, check_every_element, clear_inputs, run_allreduce, to_device, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from double_binary_tree_amd import emucomm as E
    E.lib()
    assert not E.protocol_status()
    yield
    clear_inputs()
    E.comm_destroy()
    torch.cuda.empty_cache()


def _bits(x):
    return np.ascontiguousarray(x).view(np.uint8)


def _not_abandoned():
    from double_binary_tree_amd import emucomm as E
    assert not E.protocol_status(), "an LL all-reduce was abandoned"


def _check(w, algo, count, chunk_bytes, inplace, salt=0):
    announce(f"LL {w.name} n={w.nranks} m={w.nnodes} nch={w.nchannels} algo={algo} count={count} "
             f"chunk={chunk_bytes} inplace={inplace}")
    xs = I.rank_inputs(w, count=count, salt=salt)
    want = A.allreduce(xs, w.nnodes, algo, w.nchannels, chunk_bytes, w.dtype, w.op)[0]
    got, _ = run_allreduce(xs, w.nnodes, algo, "ll", w.nchannels, chunk_bytes, w.dtype, w.op, inplace)
    _not_abandoned()
    wb = _bits(want).reshape(len(want), -1)
    for r, g in enumerate(got):
        gb = _bits(g).reshape(len(g), -1)
        if not np.array_equal(gb, wb):
            first = np.nonzero((gb != wb).any(axis=1))[0]
            raise AssertionError(f"rank {r}: {len(first)} elements differ, first at {first[:8].tolist()}")


LL_WORKLOADS = [name for name, w in I.WORKLOADS.items() if w.nranks <= 16]
CASES = [(name, algo) for name in LL_WORKLOADS for algo in ("ring", "tree")]


@pytest.mark.parametrize("name,algo", CASES)
@pytest.mark.parametrize("inplace", [False, True])
def test_ll_small_chunks(name, algo, inplace):
    # small chunks: many ring loops and tree chunks, several tasks per
    # workgroup (the ring's FIFO counters run across tasks, the tree's
    # restart at each), and a ragged tail
    w = I.WORKLOADS[name]
    unit = 16 // w.itemsize
    count = 37 * 1024 + 3 * unit + (1 if unit > 1 else 0)
    _check(w, algo, count, chunk_bytes=4096, inplace=inplace)


@pytest.mark.parametrize("name,algo", CASES)
def test_ll_workload_chunk(name, algo):
    w = I.WORKLOADS[name]
    _check(w, algo, min(w.count, 300_000 + 5), chunk_bytes=w.chunk_bytes, inplace=False, salt=1)


EDGE_COUNTS = [1, 2, 3, 7, 8, 9, 15, 16, 17, 255, 256, 257, 1023, 1024, 1025, 4099]


@pytest.mark.parametrize("algo", ["ring", "tree"])
@pytest.mark.parametrize("dtype,op", [("f32", "sum"), ("bf16", "sum"), ("f16", "max"), ("i64", "sum")])
def test_ll_edge_counts(algo, dtype, op):
    w = I.Workload("edge", 7, 6, 3, (algo,), 5, 64, dtype, op, 1,
                   ("int", -50, 50) if dtype.startswith("i") else ("normal", 1.0))
    for count in EDGE_COUNTS:
        _check(w, algo, count, chunk_bytes=64, inplace=(count % 2 == 1))


@pytest.mark.parametrize("n,m,nch", [(1, 1, 1), (2, 1, 1), (2, 2, 3), (3, 3, 2), (5, 5, 7), (12, 3, 4),
                                     (16, 16, 2), (16, 2, 5), (16, 1, 64)])
@pytest.mark.parametrize("algo", ["ring", "tree"])
def test_ll_shapes(n, m, nch, algo):
    w = I.Workload("shape", 8, n, m, (algo,), nch, 256, "f32", "sum", 1, ("normal", 1.0))
    _check(w, algo, 6 * 1024 + 13, chunk_bytes=256, inplace=False)


@pytest.mark.parametrize("algo", ["ring", "tree"])
@pytest.mark.parametrize("name", ["chain8_f32", "dtree16_bf16", "dtree15_bf16"])
def test_ll_full_size_every_element(name, algo):
    """At full size (the workload's own launch configuration), with the LL
    protocol: every element of every rank equals the oracle's, out of place
    and in place, and no call is abandoned."""
    check_every_element(I.WORKLOADS[name], algo, modes=("ll",), label="LL ")


def test_ll_communicator_runs_reduce_scatter_and_all_gather():
    """Reduce-scatter and all-gather on an LL communicator run the slot
    protocol; their results are the oracle's."""
    import torch
    from double_binary_tree_amd import emucomm as E
    from oracle import collectives as C
    w = I.Workload("coll", 8, 8, 1, ("ring",), 4, 4096, "f32", "sum", 1, ("normal", 1.0))
    block = 4096 + 4
    xs = I.rank_inputs(w, count=block * w.nranks)
    E.comm_init(w.nranks, 1, "ring", w.nchannels, w.chunk_bytes, mode="ll")
    sends = [to_device(x, "f32") for x in xs]
    outs = [torch.empty(block, dtype=torch.float32, device="cuda") for _ in range(w.nranks)]
    E.reduce_scatter_tensors(sends, outs, "sum")
    torch.cuda.synchronize()
    want = C.reduce_scatter(xs, 1, w.nchannels, w.chunk_bytes, "f32", "sum")
    for r in range(w.nranks):
        assert np.array_equal(to_host_bits(outs[r], "f32").view(np.uint8), want[r].view(np.uint8))
    gathered = [torch.empty(block * w.nranks, dtype=torch.float32, device="cuda") for _ in range(w.nranks)]
    E.all_gather_tensors(outs, gathered)
    torch.cuda.synchronize()
    cat = np.concatenate([to_host_bits(o, "f32") for o in outs])
    for g in gathered:
        assert np.array_equal(to_host_bits(g, "f32").view(np.uint8), cat.view(np.uint8))
    _not_abandoned()


@pytest.mark.parametrize("algo", ["ring", "tree"])
def test_ll_abandoned_call_is_reported_and_the_next_call_is_right(algo, monkeypatch):
    """Failure handling, forced from the host: EMU_LL_SPIN_LIMIT=0 makes
    every wait give up at its first poll that finds nothing ready, so the
    call abandons; every wave
    still meets the workgroup barriers and the kernel ends.  The status word
    reports it, and the next call (normal limit; the FIFOs live in LDS and
    restart with every launch) is bit-exact again."""
    import torch
    from double_binary_tree_amd import emucomm as E
    w = I.Workload("abandon", 9, 8, 2, (algo,), 4, 4096, "f32", "sum", 1, ("normal", 1.0))
    count = 1 << 20
    xs = I.rank_inputs(w, count=count, salt=6)
    want = A.allreduce(xs, w.nnodes, algo, w.nchannels, w.chunk_bytes, "f32", "sum")[0]
    E.comm_init(w.nranks, w.nnodes, algo, w.nchannels, w.chunk_bytes, mode="ll")
    sends = [to_device(x, "f32") for x in xs]
    recvs = [torch.empty_like(s) for s in sends]
    assert not E.protocol_status()
    abandoned = False
    for attempt in range(5):
        announce(f"LL {algo} forced abandon, attempt {attempt}")
        monkeypatch.setenv("EMU_DEBUG", "2")      # the library reads test hooks only in debug mode
        monkeypatch.setenv("EMU_LL_SPIN_LIMIT", "0")
        E.allreduce_tensors(sends, recvs, "sum")
        monkeypatch.delenv("EMU_LL_SPIN_LIMIT")
        monkeypatch.delenv("EMU_DEBUG")
        torch.cuda.synchronize()
        if E.protocol_status():
            abandoned = True
            break
    assert abandoned, "a spin limit of 0 never made a wait give up"
    assert not E.protocol_status()
    E.allreduce_tensors(sends, recvs, "sum")
    torch.cuda.synchronize()
    assert not E.protocol_status()
    for r in recvs:
        assert np.array_equal(to_host_bits(r, "f32").view(np.uint8), want.view(np.uint8))
