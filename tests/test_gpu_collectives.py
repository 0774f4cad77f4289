"""Parity of the standalone reduce-scatter and all-gather (HIP path through
the C ABI) with the oracle, bit-exact, in both modes, out of place and in
place, with identity and permuted per-channel ring orders."""

from dataclasses import replace

import numpy as np
import pytest

from double_binary_tree_amd import inputs as I
from oracle import collectives as C
from tests.gpu_util import announce, to_device, to_host_bits

pytestmark = pytest.mark.gpu

_chain = I.WORKLOADS["chain8_f32"]
# name -> (workload shape, per-channel order seed or None)
SHAPES = {
    "ring4_i32": (I.WORKLOADS["ring4_i32"], None),
    "chain8_f32": (_chain, None),
    "chain8_bf16_orders": (replace(_chain, dtype="bf16"), 201),
    "hier4x8_f16_orders": (I.WORKLOADS["hier4x8_f16"], 202),
    "hier4x8_f32max": (I.WORKLOADS["hier4x8_f32max"], None),
    "dtree16_i64": (replace(I.WORKLOADS["hier4x8_i64"], nranks=16, nnodes=16, nchannels=8), 203),
    "three_f32max": (replace(_chain, nranks=3, nchannels=5, op="max"), 204),
    "wide64_f32": (replace(_chain, nranks=64, nnodes=8, nchannels=8), 205),
    "one_f16": (replace(I.WORKLOADS["hier4x8_f16"], nranks=1, nnodes=1, nchannels=2), None),
}


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


def _intra(w, seed):
    return None if seed is None else I.intra_orders(w.nranks, w.nnodes, w.nchannels, seed)


def _same_bits(got, want, what):
    g = np.ascontiguousarray(got).view(np.uint8)
    h = np.ascontiguousarray(want).view(np.uint8)
    if not np.array_equal(g, h):
        bad = np.nonzero(g != h)[0]
        raise AssertionError(f"{what}: {len(bad)} bytes differ, first at byte {bad[:6].tolist()}")


def _reduce_scatter(name, mode, rc, chunk, inplace, salt=0):
    import torch
    from double_binary_tree_amd import emucomm as E
    w, seed = SHAPES[name]
    intra = _intra(w, seed)
    n = w.nranks
    announce(f"reduce-scatter {name} mode={mode} recvcount={rc} chunk={chunk} inplace={inplace}")
    xs = I.rank_inputs(w, count=n * rc, salt=salt)
    want = C.reduce_scatter(xs, w.nnodes, w.nchannels, chunk, w.dtype, w.op, intra=intra)
    E.comm_init(n, w.nnodes, "ring", w.nchannels, chunk, mode=mode, intra=intra)
    sends = [to_device(x, w.dtype) for x in xs]
    recvs = [s[r * rc:(r + 1) * rc] for r, s in enumerate(sends)] if inplace else \
        [torch.empty(rc, dtype=sends[0].dtype, device="cuda") for _ in range(n)]
    E.reduce_scatter_tensors(sends, recvs, w.op)
    torch.cuda.synchronize()
    for r in range(n):
        _same_bits(to_host_bits(recvs[r], w.dtype), want[r], f"rank {r}")


def _all_gather(name, mode, sc, chunk, inplace, salt=0):
    import torch
    from double_binary_tree_amd import emucomm as E
    w, seed = SHAPES[name]
    intra = _intra(w, seed)
    n = w.nranks
    announce(f"all-gather {name} mode={mode} sendcount={sc} chunk={chunk} inplace={inplace}")
    xs = I.rank_inputs(w, count=sc, salt=salt)
    want = C.all_gather(xs, w.nnodes, w.nchannels, chunk, w.dtype, intra=intra)
    E.comm_init(n, w.nnodes, "tree", w.nchannels, chunk, mode=mode, intra=intra)   # ring whatever the algo
    if inplace:
        recvs = [torch.zeros(n * sc, dtype=to_device(xs[0][:1], w.dtype).dtype, device="cuda") for _ in range(n)]
        sends = []
        for r in range(n):
            recvs[r][r * sc:(r + 1) * sc] = to_device(xs[r], w.dtype)
            sends.append(recvs[r][r * sc:(r + 1) * sc])
    else:
        sends = [to_device(x, w.dtype) for x in xs]
        recvs = [torch.full((n * sc,), 7, dtype=sends[0].dtype, device="cuda") for _ in range(n)]
    E.all_gather_tensors(sends, recvs)
    torch.cuda.synchronize()
    for r in range(n):
        _same_bits(to_host_bits(recvs[r], w.dtype), want[r], f"rank {r}")


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("mode", ["fused", "stepwise"])
@pytest.mark.parametrize("inplace", [False, True])
def test_reduce_scatter_parity(name, mode, inplace):
    unit = 16 // SHAPES[name][0].itemsize
    _reduce_scatter(name, mode, 1301 * unit, 4096, inplace)


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("mode", ["fused", "stepwise"])
@pytest.mark.parametrize("inplace", [False, True])
def test_all_gather_parity(name, mode, inplace):
    unit = 16 // SHAPES[name][0].itemsize
    _all_gather(name, mode, 1301 * unit, 4096, inplace)


@pytest.mark.parametrize("name", ["chain8_f32", "hier4x8_f16_orders", "three_f32max"])
@pytest.mark.parametrize("mode", ["fused", "stepwise"])
def test_collective_edge_counts(name, mode):
    unit = 16 // SHAPES[name][0].itemsize
    for units in (1, 2, 3, 17, 64, 65, 257):
        _reduce_scatter(name, mode, units * unit, 64, False, salt=3)
        _all_gather(name, mode, units * unit, 64, False, salt=3)


@pytest.mark.parametrize("mode", ["fused", "stepwise"])
def test_collectives_full_size(mode):
    # The all-reduce workload's shape and chunk at full size: reduce-scatter
    # of 8 blocks of 2 Mi f32 (64 MiB per rank in), all-gather of 2 Mi f32
    # per rank (64 MiB per rank out); every output byte checked.
    w, _ = SHAPES["chain8_f32"]
    rc = w.count // w.nranks
    _reduce_scatter("chain8_f32", mode, rc, w.chunk_bytes, False, salt=4)
    _all_gather("chain8_f32", mode, rc, w.chunk_bytes, False, salt=4)
