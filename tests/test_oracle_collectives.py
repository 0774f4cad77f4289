"""Pins of the reduce-scatter and all-gather oracle (CPU only)."""

import numpy as np
import pytest

from double_binary_tree_amd import inputs as I
from oracle import allreduce as A
from oracle import collectives as C
from oracle import numerics as N
from tests.conftest import golden_lines


def _pin(tag):
    vals = {}
    for line in golden_lines("order_pins_f32.txt"):
        name, kind, *nums = line.split()
        if name == tag:
            vals[kind] = [float(x) for x in nums]
    return vals


def test_reduce_scatter_float_order_pin():
    pin = _pin("RS3")
    inputs = [np.full(12, v, dtype=np.float32) for v in pin["inputs"]]
    out = C.reduce_scatter(inputs, 1, 1, 512 * 1024, "f32", "sum")
    for r in range(3):
        assert out[r].tolist() == pin[f"expect{r}"]


@pytest.mark.parametrize("n,m,nch,rc,chunk", [(1, 1, 1, 5, 16), (2, 1, 3, 37, 16), (4, 2, 2, 100, 32),
                                              (5, 5, 4, 41, 48), (8, 1, 12, 300, 64), (6, 3, 5, 64, 16)])
@pytest.mark.parametrize("op", ["sum", "max"])
def test_reduce_scatter_brute_force_integers(n, m, nch, rc, chunk, op):
    rng = np.random.default_rng(n * 31 + rc)
    xs = [rng.integers(-(1 << 31), (1 << 31) - 1, size=n * rc, dtype=np.int64).astype(np.int32) for _ in range(n)]
    out = C.reduce_scatter(xs, m, nch, chunk, "i32", op)
    for r in range(n):
        blk = [x[r * rc:(r + 1) * rc].astype(np.int64) for x in xs]
        if op == "sum":
            want = np.zeros(rc, dtype=np.int64)
            for b in blk:
                want += b
            want = ((want + (1 << 31)) % (1 << 32) - (1 << 31)).astype(np.int32)   # two's-complement wrap
        else:
            want = np.maximum.reduce(blk).astype(np.int32)
        assert np.array_equal(out[r], want), r


@pytest.mark.parametrize("n,m,nch,sc,chunk", [(1, 1, 1, 5, 16), (3, 1, 2, 37, 16), (4, 2, 3, 100, 32),
                                              (7, 7, 4, 9, 16), (8, 2, 12, 300, 64)])
def test_all_gather_is_the_concatenation(n, m, nch, sc, chunk):
    rng = np.random.default_rng(n + sc)
    xs = [rng.standard_normal(sc).astype(np.float32) for _ in range(n)]
    intra = I.intra_orders(n, m, nch, 9) if m < n else None
    out = C.all_gather(xs, m, nch, chunk, "f32", intra=intra)
    want = np.concatenate(xs)
    for r in range(n):
        assert out[r].view(np.uint32).tolist() == want.view(np.uint32).tolist()


@pytest.mark.parametrize("n,m,nch,chunk,dtype", [(3, 1, 1, 16, "f32"), (4, 2, 3, 32, "bf16"), (8, 1, 12, 64, "f16"),
                                                 (6, 3, 4, 48, "f32"), (5, 5, 2, 16, "bf16")])
@pytest.mark.parametrize("permuted", [False, True])
def test_halves_compose_to_the_ring_allreduce(n, m, nch, chunk, dtype, permuted):
    # The ring all-reduce is its reduce-scatter followed by its all-gather.
    # In the all-reduce, block k finishes at ring position k-1 (rank o[k-1]);
    # the standalone reduce-scatter gives each rank its own block.  So move
    # block k of every input to block o[k-1], reduce-scatter, all-gather, and
    # move the blocks back: the bits must be the all-reduce's (one channel,
    # N equal unit-aligned blocks, one ring loop, so the rank-chunks are the
    # blocks).
    unit = 16 // N.ITEMSIZE[dtype]
    rc = 3 * unit
    count = n * rc
    intra = I.intra_orders(n, m, 1, 17) if permuted else None
    o = intra[0] if intra else list(range(n))
    xs = I.rank_inputs(replace_workload(n, m, 1, dtype), count=count)
    ar = A.allreduce(xs, m, "ring", 1, 1 << 20, dtype, "sum", intra=intra)
    moved = [np.empty_like(x) for x in xs]
    for x, y in zip(xs, moved):
        for k in range(n):
            d = o[(k - 1) % n]
            y[d * rc:(d + 1) * rc] = x[k * rc:(k + 1) * rc]
    rs = C.reduce_scatter(moved, m, 1, 1 << 20, dtype, "sum", intra=intra)
    ag = C.all_gather(rs, m, 1, 1 << 20, dtype, intra=intra)
    for r in range(n):
        back = np.empty_like(ag[r])
        for k in range(n):
            d = o[(k - 1) % n]
            back[k * rc:(k + 1) * rc] = ag[r][d * rc:(d + 1) * rc]
        assert back.view(np.uint8).tobytes() == np.asarray(ar[r]).view(np.uint8).tobytes(), r


def replace_workload(n, m, nch, dtype):
    from dataclasses import replace
    return replace(I.WORKLOADS["chain8_f32"], nranks=n, nnodes=m, nchannels=nch, dtype=dtype)


def test_send_volumes():
    # Each half sends (N-1) blocks per rank.
    n, rc = 4, 64
    xs = [np.zeros(n * rc, dtype=np.int32) for _ in range(n)]
    st = {}
    C.reduce_scatter(xs, 1, 2, 64, "i32", "sum", stats=st)
    assert st["sent_elems"] == [(n - 1) * rc] * n
    C.all_gather([x[:rc] for x in xs], 1, 2, 64, "i32", stats=st)
    assert st["sent_elems"] == [(n - 1) * rc] * n
