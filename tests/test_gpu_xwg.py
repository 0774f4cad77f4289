"""Parity of the stepwise ring all-reduce across workgroups
(EMU_TRANSPORT_DEVICE: one workgroup per channel and ring position, steps
handed over through FIFOs in device memory) with the CPU oracle, through the
C ABI, under both protocols (SIMPLE: release fence plus tail counter; LL:
flag-in-line words).

The transport changes where a step's data waits between two positions,
never the order of any reduction, so the bar is the in-workgroup stepwise
ring's: bit-exact to the oracle for every type.  Every case also checks that
no call was abandoned (emu_protocol_status)."""

import numpy as np
import pytest

from double_binary_tree_amd import inputs as I
from oracle import allreduce as A
from tests.gpu_util import announce, check_every_element, clear_inputs, run_allreduce, to_device, to_host_bits

pytestmark = pytest.mark.gpu

MODES = ("xwg", "xwg_ll")


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
    assert not E.protocol_status(), "a cross-workgroup all-reduce was abandoned"


def _compare(got, want):
    wb = _bits(want).reshape(len(want), -1)
    for r, g in enumerate(got):
        gb = _bits(g).reshape(len(g), -1)
        if not np.array_equal(gb, wb):
            first = np.nonzero((gb != wb).any(axis=1))[0]
            raise AssertionError(f"rank {r}: {len(first)} elements differ, first at {first[:8].tolist()}")


def _check(w, mode, count, chunk_bytes, inplace, salt=0):
    announce(f"{mode} {w.name} n={w.nranks} m={w.nnodes} nch={w.nchannels} count={count} "
             f"chunk={chunk_bytes} inplace={inplace}")
    xs = I.rank_inputs(w, count=count, salt=salt)
    want = A.allreduce(xs, w.nnodes, "ring", w.nchannels, chunk_bytes, w.dtype, w.op)[0]
    got, _ = run_allreduce(xs, w.nnodes, "ring", mode, w.nchannels, chunk_bytes, w.dtype, w.op, inplace)
    _not_abandoned()
    _compare(got, want)


@pytest.mark.parametrize("name", list(I.WORKLOADS))
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("inplace", [False, True])
def test_xwg_small_chunks(name, mode, inplace):
    # 4 KiB chunks: many ring loops per channel, so the FIFO counters run
    # across loops and slots are reused many times; a ragged tail
    w = I.WORKLOADS[name]
    unit = 16 // w.itemsize
    count = 37 * 1024 + 3 * unit + (1 if unit > 1 else 0)
    _check(w, mode, count, chunk_bytes=4096, inplace=inplace)


@pytest.mark.parametrize("name", list(I.WORKLOADS))
@pytest.mark.parametrize("mode", MODES)
def test_xwg_workload_chunk(name, mode):
    w = I.WORKLOADS[name]
    _check(w, mode, min(w.count, 300_000 + 5), chunk_bytes=w.chunk_bytes, inplace=False, salt=1)


EDGE_COUNTS = [1, 2, 3, 7, 8, 9, 15, 16, 17, 255, 256, 257, 1023, 1024, 1025, 4099]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype,op", [("f32", "sum"), ("bf16", "sum"), ("f16", "max"), ("i64", "sum")])
def test_xwg_edge_counts(mode, dtype, op):
    # 64-byte chunks: blocks of a few vectors, most channels and blocks empty
    w = I.Workload("edge", 7, 6, 3, ("ring",), 5, 64, dtype, op, 1,
                   ("int", -50, 50) if dtype.startswith("i") else ("normal", 1.0))
    for count in EDGE_COUNTS:
        _check(w, mode, count, chunk_bytes=64, inplace=(count % 2 == 1))


# at most 512 workgroups (16 x 32): what the SIMPLE kernel can keep resident
@pytest.mark.parametrize("n,m,nch", [(1, 1, 1), (1, 1, 3), (2, 1, 1), (2, 2, 3), (3, 3, 2), (5, 5, 7),
                                     (12, 3, 4), (16, 1, 32), (64, 8, 4), (64, 64, 2)])
@pytest.mark.parametrize("mode", MODES)
def test_xwg_shapes(n, m, nch, mode):
    w = I.Workload("shape", 8, n, m, ("ring",), nch, 256, "f32", "sum", 1, ("normal", 1.0))
    _check(w, mode, 6 * 1024 + 13, chunk_bytes=256, inplace=False)


@pytest.mark.parametrize("mode", MODES)
def test_xwg_counters_continue_across_calls(mode):
    """One communicator, several calls of different sizes and types in a
    row (each its own plan on the same FIFOs): every call starts from the
    consumed counts the previous one left, and every result is the
    oracle's."""
    w0 = I.Workload("seq", 9, 8, 2, ("ring",), 6, 8192, "f32", "sum", 1, ("normal", 1.0))
    for i, (count, dtype, op) in enumerate([(50_001, "f32", "sum"), (3, "f32", "sum"), (120_000, "bf16", "sum"),
                                            (50_001, "f32", "sum"), (77_777, "i32", "max"), (1, "i64", "sum")]):
        w = I.Workload("seq", 9, 8, 2, ("ring",), 6, 8192, dtype, op, 1,
                       ("int", -50, 50) if dtype.startswith("i") else ("normal", 1.0))
        _check(w, mode, count, chunk_bytes=w0.chunk_bytes, inplace=(i % 2 == 1), salt=i)


@pytest.mark.parametrize("name", ["chain8_f32", "dtree16_bf16", "hier4x8_f16"])
@pytest.mark.parametrize("mode", MODES)
def test_xwg_full_size_every_element(name, mode):
    """At full size (the workload's own channels and chunk), with the FIFOs
    in device memory: every element of every rank equals the oracle's ring
    result, out of place and in place, and no call is abandoned."""
    from double_binary_tree_amd import emucomm as E
    check_every_element(I.WORKLOADS[name], "ring", modes=(mode,), label=f"{mode} ")
    assert not E.protocol_status(), "a device-transport call was abandoned"


def test_xwg_rejects_a_grid_that_cannot_be_resident():
    """64 ranks x 64 channels = 4096 workgroups: more than the device holds at
    once, so the call is refused before anything is launched."""
    import torch
    from double_binary_tree_amd import emucomm as E
    announce("xwg capacity refusal")
    E.comm_init(64, 8, "ring", 64, 4096, mode="xwg")
    bufs = [torch.zeros(64, dtype=torch.float32, device="cuda") for _ in range(64)]
    ptrs = [b.data_ptr() for b in bufs]
    rc = E.allreduce_raw(ptrs, ptrs, 64, E.DTYPE["f32"], E.OP["sum"], torch.cuda.current_stream().cuda_stream)
    assert rc == E.ERR_INVALID_ARGUMENT
    _not_abandoned()


@pytest.mark.parametrize("mode", MODES)
def test_xwg_communicator_runs_reduce_scatter_and_all_gather(mode):
    """Reduce-scatter and all-gather on such a communicator run the
    one-workgroup stepwise kernels; their results are the oracle's."""
    import torch
    from double_binary_tree_amd import emucomm as E
    from oracle import collectives as C
    w = I.Workload("coll", 8, 8, 1, ("ring",), 4, 4096, "f32", "sum", 1, ("normal", 1.0))
    block = 4096 + 4
    xs = I.rank_inputs(w, count=block * w.nranks)
    E.comm_init(w.nranks, 1, "ring", w.nchannels, w.chunk_bytes, mode=mode)
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


@pytest.mark.parametrize("mode", MODES)
def test_xwg_abandoned_call_is_reported_and_recovered(mode, monkeypatch):
    """Failure handling, forced from the host: EMU_XWG_SPIN_LIMIT=0 makes
    every wait give up at its first poll that finds nothing ready, so the
    call abandons (every
    workgroup still exits).  Until emu_protocol_status has reported it, a
    later call does nothing (the abandon word is sticky, the FIFO counters
    no longer match); the report clears the FIFOs, and the next call is
    correct again."""
    import torch
    from double_binary_tree_amd import emucomm as E
    w = I.Workload("abandon", 9, 8, 1, ("ring",), 4, 4096, "f32", "sum", 1, ("normal", 1.0))
    count = 1 << 20
    xs = I.rank_inputs(w, count=count, salt=5)
    want = A.allreduce(xs, 1, "ring", w.nchannels, w.chunk_bytes, "f32", "sum")[0]
    E.comm_init(w.nranks, 1, "ring", w.nchannels, w.chunk_bytes, mode=mode)
    sends = [to_device(x, "f32") for x in xs]
    recvs = [torch.empty_like(s) for s in sends]
    assert not E.protocol_status()
    abandoned = False
    for attempt in range(5):
        announce(f"{mode} forced abandon, attempt {attempt}")
        monkeypatch.setenv("EMU_DEBUG", "2")      # the library reads test hooks only in debug mode
        monkeypatch.setenv("EMU_XWG_SPIN_LIMIT", "0")
        E.allreduce_tensors(sends, recvs, "sum")
        monkeypatch.delenv("EMU_XWG_SPIN_LIMIT")
        monkeypatch.delenv("EMU_DEBUG")
        torch.cuda.synchronize()
        for r in recvs:
            r.fill_(-7.0)
        E.allreduce_tensors(sends, recvs, "sum")      # normal limit
        torch.cuda.synchronize()
        if E.protocol_status():
            # the second call found the abandon word set and left the outputs alone
            for r in recvs:
                assert bool((r == -7.0).all()), "a call after an abandoned one wrote its outputs"
            abandoned = True
            break
        # neither call abandoned: both completed, and the outputs are right
        assert np.array_equal(to_host_bits(recvs[0], "f32").view(np.uint8), want.view(np.uint8))
    assert abandoned, "a spin limit of 0 never made a wait give up"
    assert not E.protocol_status()
    E.allreduce_tensors(sends, recvs, "sum")
    torch.cuda.synchronize()
    assert not E.protocol_status()
    for r in recvs:
        assert np.array_equal(to_host_bits(r, "f32").view(np.uint8), want.view(np.uint8))
