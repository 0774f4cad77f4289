"""Host-side checks of libemucomm (no GPU): the library loads, exports every
function include/emu_comm.h declares, builds the same tree records as the
oracle topology, and rejects bad arguments before touching a device."""

import os
import re

import pytest

from double_binary_tree_amd import emucomm as E
from oracle import topology as T
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "emu_comm.h")


@pytest.fixture(autouse=True)
def _fresh():
    E.comm_destroy()
    yield
    E.comm_destroy()


def test_exports_every_declared_function():
    text = open(HEADER, encoding="utf-8").read()
    names = re.findall(r"^\s*(?:int|const char\s*\*)\s*(emu_\w+)\s*\(", text, flags=re.M)
    assert len(names) >= 6
    L = E.lib()
    for name in names:
        assert hasattr(L, name), name


def test_header_constants_match_binding():
    text = open(HEADER, encoding="utf-8").read()
    consts = dict(re.findall(r"#define\s+(EMU_\w+)\s+(0x[0-9A-Fa-f]+|\d+)", text))
    val = {k: int(v, 0) for k, v in consts.items()}
    assert val["EMU_ALGO_RING"] == E.ALGO["ring"] and val["EMU_ALGO_TREE"] == E.ALGO["tree"]
    assert val["EMU_ALGO_AUTO"] == E.ALGO["auto"]
    assert [val[f"EMU_PATTERN_{k}"] for k in ("TREE", "SPLIT_TREE", "BALANCED_TREE")] == \
        [E.PATTERNS[k] for k in ("tree", "split", "balanced")]
    assert val["EMU_MODE_FUSED"] == E.MODE["fused"] and val["EMU_MODE_STEPWISE"] == E.MODE["stepwise"]
    assert val["EMU_PROTO_LL"] == E.MODE["ll"] and val["EMU_PROTO_SIMPLE"] == 0
    assert val["EMU_TRANSPORT_DEVICE"] == E.MODE["xwg"] and E.MODE["xwg_ll"] == E.MODE["xwg"] | E.MODE["ll"]
    for k, name in (("EMU_INT32", "i32"), ("EMU_INT64", "i64"), ("EMU_FLOAT32", "f32"),
                    ("EMU_FLOAT16", "f16"), ("EMU_BFLOAT16", "bf16")):
        assert val[k] == E.DTYPE[name]
    assert val["EMU_SUM"] == E.OP["sum"] and val["EMU_MAX"] == E.OP["max"]


def _shapes():
    for n in range(1, 65):
        for m in range(1, n + 1):
            if n % m == 0 and (n <= 12 or m in (1, 2, 3, 4, n // 8 if n % 8 == 0 else 1, n)):
                yield n, m


def test_topology_matches_oracle():
    checked = 0
    for n, m in _shapes():
        for nch in (1, 2, 5, 16):
            E.comm_init(n, m, "tree", nch, 1 << 19)
            ref = T.build_topology(n, m, nch)
            assert E.tree_depth() == ref.channels[0].depth
            for c in range(nch):
                for r in range(n):
                    up, down = E.tree_topology(c, r)
                    assert up == ref.channels[c].up[r], (n, m, nch, c, r)
                    assert down == ref.channels[c].down[r], (n, m, nch, c, r)
                    checked += 1
    assert checked > 20000


def test_ring_comm_also_reports_topology():
    E.comm_init(8, 1, "ring", 12, 1 << 19, mode="fused")
    assert E.tree_topology(0, 0) == (-1, [1, -1, -1])
    assert E.tree_topology(11, 7) == (6, [-1, -1, -1])


def _orders(rng, n, m, nch):
    L = n // m
    return [[int(r) for node in range(m) for r in rng.permutation(range(node * L, (node + 1) * L))]
            for _ in range(nch)]


@pytest.mark.parametrize("pattern", ["tree", "split", "balanced"])
def test_graph_topology_matches_oracle(pattern):
    import numpy as np
    rng = np.random.default_rng(7)
    for n, m, nch in ((4, 2, 2), (6, 3, 4), (8, 2, 5), (12, 4, 3), (32, 4, 16), (64, 8, 8), (30, 5, 6),
                      (18, 9, 2), (4, 1, 12), (3, 1, 2)):
        for intra in (None, _orders(rng, n, m, nch)):
            E.comm_init(n, m, "tree", nch, 1 << 19, pattern=pattern, intra=intra)
            ref = T.build_topology(n, m, nch, pattern, intra)
            for c in range(nch):
                for r in range(n):
                    assert E.tree_topology(c, r) == (ref.channels[c].up[r], ref.channels[c].down[r]), \
                        (pattern, n, m, c, r)


def test_graph_table_chains():
    # The per-channel chains of the pages' 4-GPU table (12 channels, 3 orders).
    order = {0: [0, 1, 2, 3], 1: [0, 1, 2, 3], 6: [0, 1, 2, 3], 7: [0, 1, 2, 3],
             2: [0, 2, 1, 3], 3: [0, 2, 1, 3], 8: [0, 2, 1, 3], 9: [0, 2, 1, 3],
             4: [1, 0, 3, 2], 5: [1, 0, 3, 2], 10: [1, 0, 3, 2], 11: [1, 0, 3, 2]}
    intra = [order[c] for c in range(12)]
    E.comm_init(4, 1, "tree", 12, 1 << 19, mode="fused", intra=intra)
    for c in range(12):
        o = order[c]
        for i, r in enumerate(o):
            up, down = E.tree_topology(c, r)
            assert up == (o[i - 1] if i else -1)
            assert down == [o[i + 1] if i < 3 else -1, -1, -1]


def test_init_graph_rejects_bad_graphs_and_keeps_state():
    E.comm_init(4, 2, "tree", 2, 1 << 19)
    raw = E.comm_init_graph_raw
    assert raw(4, 4, 1, 2, 1 << 19, 1) == E.ERR_INVALID_ARGUMENT          # split, one rank per node
    assert raw(4, 4, 1, 2, 1 << 19, 2) == E.ERR_INVALID_ARGUMENT          # balanced, one rank per node
    assert raw(4, 1, 1, 1, 1 << 19, 3) == E.ERR_INVALID_ARGUMENT          # unknown pattern
    assert raw(4, 1, 1, 1, 1 << 19, -1) == E.ERR_INVALID_ARGUMENT
    assert raw(4, 2, 1, 1, 1 << 19, 0, [[0, 2, 1, 3]]) == E.ERR_INVALID_ARGUMENT   # rank 2 on node 1
    assert raw(4, 1, 1, 1, 1 << 19, 0, [[0, 1, 1, 3]]) == E.ERR_INVALID_ARGUMENT   # repeated rank
    assert raw(4, 1, 1, 1, 1 << 19, 0, [[0, 1, 2, 4]]) == E.ERR_INVALID_ARGUMENT   # out of range
    assert raw(4, 1, 1, 1, 1 << 19, 0, [[0, 1, 2, -1]]) == E.ERR_INVALID_ARGUMENT
    assert raw(4, 1, 7, 1, 1 << 19, 0) == E.ERR_INVALID_ARGUMENT          # algo
    up, down = E.tree_topology(0, 2)
    ref = T.build_topology(4, 2, 2).channels[0]
    assert (up, down) == (ref.up[2], ref.down[2])
    # the plain init is the graph init with the tree pattern and identity orders
    assert raw(4, 2, 1, 2, 1 << 19, 0) == E.SUCCESS
    assert (E.tree_topology(0, 2)) == (ref.up[2], ref.down[2])
    with pytest.raises(ValueError):
        E.comm_init(4, 1, "tree", 2, 1 << 19, intra=[[0, 1, 2, 3]])       # one row per channel


def test_init_rejects_bad_arguments_and_keeps_state():
    E.comm_init(4, 2, "tree", 2, 1 << 19)
    bad = [
        (0, 1, 1, 1, 1 << 19), (65, 1, 1, 1, 1 << 19), (4, 3, 1, 1, 1 << 19), (4, 0, 1, 1, 1 << 19),
        (4, 1, 1, 0, 1 << 19), (4, 1, 1, 65, 1 << 19), (4, 1, 1, 1, 0), (4, 1, 1, 1, 24), (4, 1, 1, 1, (1 << 30) + 16),
        (4, 1, 7, 1, 1 << 19), (4, 1, 0x401, 1, 1 << 19),
        # LL: stepwise only, at most 16 ranks
        (4, 1, 0x301, 1, 1 << 19), (17, 1, 0x201, 1, 1 << 19), (32, 4, 0x200, 16, 1 << 19),
        # device transport: stepwise ring only; unknown flag bits
        (4, 1, 0x401, 1, 1 << 19), (4, 1, 0x402, 1, 1 << 19), (4, 1, 0x500, 1, 1 << 19),
        (4, 1, 0x601, 1, 1 << 19), (4, 1, 0x700, 1, 1 << 19), (4, 1, 0x800, 1, 1 << 19),
    ]
    for args in bad:
        assert E.comm_init_raw(*args) == E.ERR_INVALID_ARGUMENT, args
    # the previous communicator is still active
    up, down = E.tree_topology(0, 2)
    ref = T.build_topology(4, 2, 2).channels[0]
    assert (up, down) == (ref.up[2], ref.down[2])


def test_ll_init_accepts_up_to_16_ranks():
    for n, m, algo in ((16, 1, "ring"), (16, 16, "tree"), (2, 2, "auto"), (1, 1, "tree")):
        E.comm_init(n, m, algo, 4, 1 << 19, mode="ll")
        up, down = E.tree_topology(0, n - 1)
        ref = T.build_topology(n, m, 4).channels[0]
        assert (up, down) == (ref.up[n - 1], ref.down[n - 1])


def test_device_transport_init_accepts_ring_with_any_rank_count():
    # the LL protocol over device FIFOs has no 16-rank limit
    for n, m, mode in ((64, 8, "xwg"), (64, 8, "xwg_ll"), (1, 1, "xwg"), (17, 1, "xwg_ll")):
        E.comm_init(n, m, "ring", 4, 1 << 19, mode=mode)
        up, down = E.tree_topology(0, n - 1)
        ref = T.build_topology(n, m, 4).channels[0]
        assert (up, down) == (ref.up[n - 1], ref.down[n - 1])


def test_buffer_layout():
    # buffer i at i * slot, slot = bytes rounded up to 64 KiB plus 6 KiB:
    # consecutive buffers start 6 KiB apart modulo 64 KiB (32 distinct
    # positions before the pattern repeats)
    for nbufs, nbytes in ((1, 0), (2, 1), (64, 16 << 20), (17, (64 << 10) + 1), (3, 4096)):
        offs, pool = E.buffer_layout(nbufs, nbytes)
        slot = -(-nbytes // (64 << 10)) * (64 << 10) + 6144
        assert offs == [i * slot for i in range(nbufs)] and pool == nbufs * slot
        assert all(offs[i] + nbytes <= offs[i + 1] for i in range(nbufs - 1))
        residues = [o % (64 << 10) for o in offs[:32]]
        assert len(set(residues)) == len(residues)
    L = E.lib()
    import ctypes
    arr = (ctypes.c_size_t * 4)()
    size = ctypes.c_size_t(0)
    assert L.emu_buffer_layout(0, 16, arr, ctypes.byref(size)) == E.ERR_INVALID_ARGUMENT
    assert L.emu_buffer_layout(4, 16, None, ctypes.byref(size)) == E.ERR_INVALID_ARGUMENT
    assert L.emu_buffer_layout(4, 16, arr, None) == E.ERR_INVALID_ARGUMENT
    assert L.emu_buffer_layout(4, (1 << 64) - 1, arr, ctypes.byref(size)) == E.ERR_INVALID_ARGUMENT
    assert L.emu_buffer_layout(1 << 60, 1 << 20, arr, ctypes.byref(size)) == E.ERR_INVALID_ARGUMENT


def test_calls_before_init():
    assert E.allreduce_raw([16], [32], 4, 0, 0) == E.ERR_NOT_INITIALIZED
    with pytest.raises(E.EmuError) as ei:
        E.tree_topology(0, 0)
    assert ei.value.code == E.ERR_NOT_INITIALIZED
    assert E.lib().emu_tree_depth(None) == E.ERR_NOT_INITIALIZED


def test_topology_argument_errors():
    E.comm_init(4, 1, "tree", 2, 1 << 19)
    for c, r in ((-1, 0), (2, 0), (0, -1), (0, 4)):
        with pytest.raises(E.EmuError) as ei:
            E.tree_topology(c, r)
        assert ei.value.code == E.ERR_INVALID_ARGUMENT


def test_allreduce_argument_errors_without_gpu():
    # All of these are rejected before any device call, so they run on CPU.
    E.comm_init(2, 1, "ring", 1, 1 << 19, mode="fused")
    base = 1 << 32
    ok_send, ok_recv = [base, base + 4096], [base + 8192, base + 12288]
    raw = E.allreduce_raw
    assert raw(ok_send, ok_recv, 16, 9, 0) == E.ERR_INVALID_ARGUMENT          # dtype
    assert raw(ok_send, ok_recv, 16, 2, 5) == E.ERR_INVALID_ARGUMENT          # op
    assert raw([base + 8, base + 4096], ok_recv, 16, 2, 0) == E.ERR_INVALID_ARGUMENT  # alignment
    assert raw([0, base + 4096], ok_recv, 16, 2, 0) == E.ERR_INVALID_ARGUMENT         # null
    # rank 1's send overlaps rank 0's send
    assert raw([base, base + 16], ok_recv, 16, 2, 0) == E.ERR_INVALID_ARGUMENT
    # a receive buffer partly overlapping its own send buffer
    assert raw(ok_send, [base + 16, base + 12288], 16, 2, 0) == E.ERR_INVALID_ARGUMENT
    # count 0 is a no-op, in place is fine
    assert raw(ok_send, ok_recv, 0, 2, 0) == E.SUCCESS
    assert raw(ok_send, ok_send, 0, 2, 0) == E.SUCCESS
    # absurd count
    assert raw(ok_send, ok_recv, 1 << 62, 2, 0) == E.ERR_INVALID_ARGUMENT


def test_strerror_total():
    for code in range(-1, 7):
        assert isinstance(E.strerror(code), str) and E.strerror(code)


def test_collective_argument_errors_without_gpu():
    # Reduce-scatter / all-gather checks run before any device call.
    E.comm_init(2, 1, "tree", 2, 1 << 19, mode="fused")
    base = 1 << 32
    rc = 1024                      # f32: 4 KiB blocks
    send = [base, base + 16384]    # 2 blocks each
    recv = [base + 32768, base + 36864]
    rs, ag = E.reduce_scatter_raw, E.all_gather_raw
    assert rs(send, recv, 0, 2, 0) == E.SUCCESS
    assert ag(recv, send, 0, 2) == E.SUCCESS
    assert rs(send, recv, 3, 2, 0) == E.ERR_INVALID_ARGUMENT        # 12-byte blocks are not 16-byte aligned
    assert ag(recv, send, 5, 3) == E.ERR_INVALID_ARGUMENT           # 10-byte blocks
    assert rs(send, recv, rc, 9, 0) == E.ERR_INVALID_ARGUMENT       # dtype
    assert rs(send, recv, rc, 2, 7) == E.ERR_INVALID_ARGUMENT       # op
    assert rs([base + 8, base + 16384], recv, rc, 2, 0) == E.ERR_INVALID_ARGUMENT   # alignment
    # rank 1's send (2 blocks) overlaps rank 0's send
    assert rs([base, base + 4096], recv, rc, 2, 0) == E.ERR_INVALID_ARGUMENT
    # all-gather output (2 blocks) overlapping another rank's output
    assert ag(send, [base + 32768, base + 36864], rc, 2) == E.ERR_INVALID_ARGUMENT
    # in place is recognised, any other partial overlap is not
    assert rs(send, [base + 4096, base + 16384], 0, 2, 0) == E.SUCCESS
    assert rs(send, [base + 16, base + 16384 + 4096], rc, 2, 0) == E.ERR_INVALID_ARGUMENT
    assert rs([base, base + 16384], [base + 16, base + 16384 + 4096 + 16], rc, 2, 0) == E.ERR_INVALID_ARGUMENT
    # absurd counts
    assert rs(send, recv, 1 << 60, 2, 0) == E.ERR_INVALID_ARGUMENT
    assert ag(send, recv, 1 << 60, 2) == E.ERR_INVALID_ARGUMENT


CLASS_RANKS = (8, 16, 32)       # one rank count inside each rank-count class of the cost model
_defaults = {}


def _snapshot_cost():
    if not _defaults:
        for mode in ("stepwise", "fused"):
            for algo in ("ring", "tree"):
                for n in CLASS_RANKS:
                    _defaults[(mode, algo, n)] = E.get_cost_model(algo, mode, n)
    return _defaults


def _restore_cost():
    for (mode, algo, n), (a, b) in _snapshot_cost().items():
        E.set_cost_model_ranks(algo, mode, n, a, b)


@pytest.mark.parametrize("n,m,nch", [(8, 1, 12), (16, 16, 8), (15, 15, 8), (32, 4, 16), (4, 2, 2), (64, 8, 8)])
@pytest.mark.parametrize("mode", ["stepwise", "fused"])
def test_cost_model_predictions_and_selection_match_the_oracle(n, m, nch, mode):
    # Predicted times and the AUTO choice equal the oracle's formulas and
    # selection rule (both in double precision, same operation order).
    from oracle import costmodel as CM
    _restore_cost()
    try:
        E.comm_init(n, m, "auto", nch, 1 << 19, mode=mode)
        depth = max(ch.true_depth() for ch in T.build_topology(n, m, nch).channels)
        for params in (None, ((2.0, 400000.0), (0.5, 90000.0))):
            if params is not None:
                E.set_cost_model("ring", mode, *params[0])
                E.set_cost_model("tree", mode, *params[1])
            ring = E.get_cost_model("ring", mode, n) if params is None else params[0]
            tree = E.get_cost_model("tree", mode, n) if params is None else params[1]
            for dtype, esz in (("f32", 4), ("bf16", 2), ("i64", 8)):
                for count in [0, 1, 7, 1000, 1 << 12, 1 << 16, 123457, 1 << 20, 1 << 24, 3 << 26]:
                    s = float(count) * esz
                    assert E.predict_us("ring", mode, count, dtype) == CM.ring_time(n, s, *ring)
                    assert E.predict_us("tree", mode, count, dtype) == CM.tree_time(depth, s, *tree)
                    assert E.select_algo(count, dtype) == CM.select(n, depth, s, ring + (0.0,), tree + (0.0,))
    finally:
        _restore_cost()


def test_cost_model_classes_by_rank_count():
    # The parameters of one rank-count class apply to every communicator of
    # that class and to no other: N <= 11, 12 <= N <= 22, N >= 23.
    _restore_cost()
    try:
        E.set_cost_model_ranks("ring", "stepwise", 16, 3.25, 12345.0)
        for n in (1, 8, 11, 12, 16, 22, 23, 32, 64):
            got = E.get_cost_model("ring", "stepwise", n)
            assert (got == (3.25, 12345.0)) == (12 <= n <= 22), n
            E.comm_init(n, 1, "auto", 2, 1 << 19)
            want = 2 * (n - 1) * got[0] + 2.0 * (n - 1) / n * 4000.0 / got[1]
            assert E.predict_us("ring", "stepwise", 1000, "f32") == want
        E.set_cost_model("tree", "fused", 1.5, 5000.0)       # every class
        for n in CLASS_RANKS:
            assert E.get_cost_model("tree", "fused", n) == (1.5, 5000.0)
        L = E.lib()
        import ctypes
        a, b = ctypes.c_double(), ctypes.c_double()
        assert L.emu_set_cost_model_ranks(0, 65, 1.0, 1.0) == E.ERR_INVALID_ARGUMENT
        assert L.emu_set_cost_model_ranks(0, -1, 1.0, 1.0) == E.ERR_INVALID_ARGUMENT
        assert L.emu_get_cost_model(0, 0, ctypes.byref(a), ctypes.byref(b)) == E.ERR_INVALID_ARGUMENT
        assert L.emu_get_cost_model(2, 8, ctypes.byref(a), ctypes.byref(b)) == E.ERR_INVALID_ARGUMENT
        assert L.emu_get_cost_model(0, 8, None, ctypes.byref(b)) == E.ERR_INVALID_ARGUMENT
    finally:
        _restore_cost()


def test_fixed_algorithm_is_reported_and_cost_model_errors():
    _restore_cost()
    E.comm_init(8, 1, "tree", 12, 1 << 19)
    assert E.select_algo(1 << 24, "f32") == "tree"
    E.comm_init(8, 1, "ring", 12, 1 << 19, mode="fused")
    assert E.select_algo(16, "f32") == "ring"
    L = E.lib()
    for bad in ((7, 1.0, 1.0), (2, 1.0, 1.0), (0, -1.0, 1.0), (0, 1.0, 0.0), (0, float("nan"), 1.0), (0x201, 1.0, 1.0)):
        assert L.emu_set_cost_model(*bad) == E.ERR_INVALID_ARGUMENT, bad
    import ctypes
    out = ctypes.c_double()
    assert L.emu_predict_us(2, 10, 2, ctypes.byref(out)) == E.ERR_INVALID_ARGUMENT    # AUTO has no formula
    assert L.emu_predict_us(0, 10, 9, ctypes.byref(out)) == E.ERR_INVALID_ARGUMENT
    assert L.emu_predict_us(0, 10, 2, None) == E.ERR_INVALID_ARGUMENT
    assert L.emu_select_algo(10, 2, None) == E.ERR_INVALID_ARGUMENT


def test_c_abi_check_library_is_built():
    """The plain-C ABI check (run on the GPU by tests/test_gpu_capi.py) is
    built and links the library; nothing is called here."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "host", "libcapi_check.so")
    lib = ctypes.CDLL(path)
    assert hasattr(lib, "capi_check")
