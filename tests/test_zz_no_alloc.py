"""The allocation-free all-reduce (emu_allreduce_noalloc) against the
allocating one (emu_allreduce), through the C ABI: the same bits on the same
inputs, for two calls in a row with the second one smaller, in every mode it
supports, in and out of place; and no device allocation by the library at
any point (emu_device_memory stays at zero from a fresh communicator)."""

import numpy as np
import pytest

from double_binary_tree_amd import inputs as I
from oracle import allreduce as A
from tests.gpu_util import announce, to_device, to_host_bits

pytestmark = pytest.mark.gpu

# (workload, algo, mode, first count, second count)
CASES = [
    ("chain8_f32", "ring", "fused", 1 << 20, 37 * 1024 + 5),
    ("chain8_f32", "tree", "fused", 1 << 20, 4099),
    ("chain8_f32", "ring", "stepwise", 1 << 20, 37 * 1024 + 5),
    ("chain8_f32", "tree", "stepwise", 1 << 20, 4099),
    ("chain8_f32", "ring", "ll", 300001, 1027),
    ("dtree16_bf16", "tree", "ll", 300001, 1027),
    ("dtree15_bf16", "tree", "fused", 1 << 20, 9001),
    ("dtree15_bf16", "tree", "stepwise", 1 << 20, 9001),
    ("hier4x8_f16", "tree", "stepwise", 1 << 19, 20003),
    ("hier4x8_i64", "tree", "fused", 1 << 19, 20003),
    ("hier4x8_f32max", "ring", "stepwise", 1 << 19, 20003),
    # the balanced plans: the stepwise tree in short pieces (24 MiB per rank),
    # the stepwise ring with one workgroup per task (112 MiB per rank), each
    # followed by a smaller call on the other plan
    ("chain8_f32", "tree", "stepwise", (3 << 21) + 37, 1 << 20),
    ("chain8_f32", "ring", "stepwise", (28 << 20) + 5, 1 << 20),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from double_binary_tree_amd import emucomm as E
    E.lib()
    yield
    E.comm_destroy()
    torch.cuda.empty_cache()


def _run(E, fn, sends, recvs, op):
    import torch
    dt = E.torch_dtype_name(sends[0])
    fn([t.data_ptr() for t in sends], [t.data_ptr() for t in recvs], sends[0].numel(), dt, op,
       torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("name,algo,mode,count1,count2", CASES)
@pytest.mark.parametrize("inplace", [False, True])
def test_noalloc_equals_allocating_entry_point(name, algo, mode, count1, count2, inplace):
    import torch
    from double_binary_tree_amd import emucomm as E
    w = I.WORKLOADS[name]
    announce(f"noalloc {name} {algo} {mode} inplace={inplace} counts {count1},{count2}")
    E.comm_destroy()
    assert E.device_memory() == (0, 0)
    E.comm_init(w.nranks, w.nnodes, algo, w.nchannels, w.chunk_bytes, mode=mode)
    for count in (count1, count2):
        xs = I.rank_inputs(w, count=count, salt=11)
        sends = [to_device(x, w.dtype) for x in xs]
        if inplace:
            got = [s.clone() for s in sends]
            _run(E, E.allreduce_noalloc, got, got, w.op)
        else:
            got = [torch.empty_like(s) for s in sends]
            _run(E, E.allreduce_noalloc, sends, got, w.op)
        torch.cuda.synchronize()
        assert E.device_memory() == (0, 0), "the no-allocation entry point allocated device memory"
        ref = [torch.empty_like(s) for s in sends]
        _run(E, E.allreduce, sends, ref, w.op)
        torch.cuda.synchronize()
        for r in range(w.nranks):
            assert torch.equal(got[r].view(torch.uint8), ref[r].view(torch.uint8)), \
                f"count {count} rank {r}: no-allocation result differs from emu_allreduce"
        if mode == "ll":
            assert not E.protocol_status()
        del sends, got, ref
        # back to no library allocations for the next call
        E.comm_destroy()
        E.comm_init(w.nranks, w.nnodes, algo, w.nchannels, w.chunk_bytes, mode=mode)
        assert E.device_memory() == (0, 0)


@pytest.mark.parametrize("mode", ["fused", "stepwise"])
def test_noalloc_shapes_alternate_and_match_the_oracle(mode):
    """Three shapes in turn (big, small, big again, then a second dtype) on
    one stream: each call restages the scratch tables it needs, and every
    result equals the oracle's on every element."""
    import torch
    from double_binary_tree_amd import emucomm as E
    w = I.WORKLOADS["chain8_f32"]
    E.comm_destroy()
    E.comm_init(w.nranks, w.nnodes, "tree", 3, 4096, mode=mode)
    for count, salt in ((50001, 1), (777, 2), (50001, 3), (4097, 4)):
        announce(f"noalloc alternate {mode} count {count}")
        xs = I.rank_inputs(w, count=count, salt=salt)
        want = A.allreduce(xs, w.nnodes, "tree", 3, 4096, w.dtype, w.op)
        sends = [to_device(x, w.dtype) for x in xs]
        recvs = [torch.empty_like(s) for s in sends]
        _run(E, E.allreduce_noalloc, sends, recvs, w.op)
        torch.cuda.synchronize()
        for r in range(w.nranks):
            assert np.array_equal(to_host_bits(recvs[r], w.dtype).view(np.uint8), want[r].view(np.uint8)), \
                f"count {count} rank {r}"
    assert E.device_memory() == (0, 0)
    E.comm_destroy()
