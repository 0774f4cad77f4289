"""Host planner checks (CPU only): the library's tiles, fused order tables,
stepwise tasks and compiled tree programs, dumped by a small C++ driver
built from the host-only planner sources with AddressSanitizer and
UndefinedBehaviorSanitizer, are compared with the oracle's partition,
ring orders and tree folds."""

import json
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import numerics as N
from oracle import partition as P
from oracle import topology as T
from oracle import tree as TR
from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "double_binary_tree_amd", "csrc")
BUILD = os.path.join(ROOT, "_build", "host_tests")
EXE = os.path.join(BUILD, "planner_dump")
PATTERN_NAMES = ("tree", "split", "balanced")


@pytest.fixture(scope="module")
def dump():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    os.makedirs(BUILD, exist_ok=True)
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I" + CSRC, os.path.join(ROOT, "tests", "host", "planner_dump.cpp"),
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "topology.cpp"), "-o", EXE + f".{os.getpid()}"]
    subprocess.run(cmd, check=True, capture_output=True)
    os.replace(EXE + f".{os.getpid()}", EXE)   # atomic: parallel workers may run the previous build
    cache = {}

    def run(n, m, nch, chunk_bytes, esz, count, pattern=0, intra=None):
        arg = "-" if intra is None else ",".join(str(r) for row in intra for r in row)
        key = (n, m, nch, chunk_bytes, esz, count, pattern, arg)
        if key not in cache:
            env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1")
            out = subprocess.run([EXE, str(n), str(m), str(nch), str(chunk_bytes), str(esz), str(count),
                                  str(pattern), arg], check=True, capture_output=True, text=True, env=env)
            cache[key] = json.loads(out.stdout)
        return cache[key]
    return run


def _orders(n, m, nch, seed):
    """Random per-channel orders (node by node), drawn from a pool of three so
    that some channels share an order."""
    if seed is None:
        return None
    rng = np.random.default_rng(seed)
    L = n // m
    pool = []
    for _ in range(3):
        row = []
        for node in range(m):
            row += [int(x) for x in rng.permutation(range(node * L, (node + 1) * L))]
        pool.append(row)
    return [pool[int(rng.integers(0, len(pool)))] for _ in range(nch)]


CASES = [(4, 1, 1, 512 * 1024, 4, 1024), (8, 1, 12, 4096, 4, 37 * 1024 + 5), (16, 16, 8, 1024, 2, 20000),
         (15, 15, 8, 1024, 2, 20003), (32, 4, 16, 2048, 2, 30001), (32, 4, 16, 2048, 8, 9000),
         (6, 3, 5, 64, 8, 1025), (3, 3, 2, 16, 4, 257), (1, 1, 1, 64, 4, 100), (64, 8, 64, 256, 4, 6157),
         (2, 2, 3, 64, 2, 7), (12, 3, 4, 512, 4, 0), (5, 5, 7, 48, 4, 9)]
# (n, m, nch, chunk, esz, count, pattern, order seed): per-channel orders and head patterns
GRAPH_CASES = [(4, 1, 12, 1024, 4, 20000, 0, 1), (8, 2, 6, 512, 4, 9001, 1, None), (8, 2, 6, 512, 2, 9001, 2, 2),
               (6, 3, 4, 256, 4, 3001, 1, 3), (32, 4, 16, 2048, 2, 30001, 2, 4), (12, 4, 5, 64, 8, 2049, 1, 5),
               (64, 8, 8, 256, 4, 6157, 1, 6), (3, 1, 2, 16, 4, 257, 0, 7), (8, 1, 1, 4096, 4, 5000, 0, 8)]
ALL = [c + (0, None) for c in CASES] + GRAPH_CASES


def _topo(n, m, nch, pattern, seed):
    return T.build_topology(n, m, nch, PATTERN_NAMES[pattern], _orders(n, m, nch, seed))


def _dump(dump, n, m, nch, chunk, esz, count, pattern, seed):
    return dump(n, m, nch, chunk, esz, count, pattern, _orders(n, m, nch, seed))


def _covers(pieces, count):
    pos = 0
    for start, n in pieces:
        assert start == pos and n > 0, (start, n, pos)
        pos += n
    assert pos == count


def _decode(fo, variant, n):
    """Input ranks and (program mode) register words of a fused variant."""
    if fo["mode"] == 0:
        return [fo["rotate_perm"][(variant + j) % n] for j in range(n)], None
    row, k = variant >> 8, variant & 0xFF
    ent = fo["rows"][row * 128 + k: row * 128 + k + n]
    return [e & 0xFF for e in ent], ([e >> 8 for e in ent] if fo["mode"] == 2 else None)


def _run_program(prog, xs, dtype, op):
    """Evaluate a compiled register program on the oracle's arithmetic."""
    regs = [None] * 8
    for rank, w in zip(prog["perm"], prog["instr"]):
        dreg = (w >> 1) & 7
        regs[dreg] = N.combine(dtype, op, regs[dreg], xs[rank]) if w & 1 else xs[rank].copy()
        for p_ in range(1, (w >> 4) + 1):
            regs[dreg - p_] = N.combine(dtype, op, regs[dreg - p_], regs[dreg - p_ + 1])
    return regs[0]


def _fold(seq, words, xs, dtype):
    """Evaluate a decoded fused order on the oracle's arithmetic."""
    if words is None:
        acc = xs[seq[0]].copy()
        for r in seq[1:]:
            acc = N.combine(dtype, "sum", acc, xs[r])
        return acc
    return _run_program({"perm": seq, "instr": words}, xs, dtype, "sum")


def _inputs(n, esz, seed):
    rng = np.random.default_rng(seed)
    dtype = {2: "bf16", 4: "f32", 8: "i64"}[esz]
    if dtype == "i64":
        return dtype, [rng.integers(-1 << 40, 1 << 40, size=64) for _ in range(n)]
    xs = [rng.standard_normal(64).astype(np.float32) for _ in range(n)]
    return dtype, ([N.f32_to_bf16(x) for x in xs] if dtype == "bf16" else xs)


def _bits(a):
    return np.asarray(a).view(np.uint8).tobytes()


def _oracle_tree_fold(ch, xs, dtype):
    return TR.tree_allreduce_chunk(xs, ch.up, ch.down, lambda a, b: N.combine(dtype, "sum", a, b),
                                   lambda a: a.copy())[0]


@pytest.mark.parametrize("n,m,nch,chunk,esz,count,pattern,seed", ALL)
def test_fused_tiles_and_orders_follow_the_oracle(dump, n, m, nch, chunk, esz, count, pattern, seed):
    d = _dump(dump, n, m, nch, chunk, esz, count, pattern, seed)
    unit = 16 // esz
    topo = _topo(n, m, nch, pattern, seed)
    assert d["nrings"] == len({tuple(ch.order) for ch in topo.channels})
    assert d["ntrees"] == len({(tuple(ch.up), tuple(map(tuple, ch.down))) for ch in topo.channels})
    # per element: channel and (ring) rank-chunk index
    chan = np.full(count, -1, dtype=np.int64)
    kidx = np.full(count, -1, dtype=np.int64)
    for c, (off, ln) in enumerate(P.channel_ranges(count, unit, nch)):
        chan[off:off + ln] = c
        for blocks in P.ring_loops(off, ln, n, chunk // esz, unit):
            for k, (o, b) in enumerate(blocks):
                kidx[o:o + b] = k
    dtype, xs = _inputs(n, esz, n * 7 + m)
    for key in ("fused_ring", "fused_tree"):
        fo = d[key]
        assert "error" not in fo
        tiles = fo["tiles"]
        _covers([(s_, ln) for s_, ln, _ in tiles], count)
        checked = set()
        for s_, ln, v in tiles:
            assert ln <= 256 * unit
            if ln == 256 * unit:
                assert s_ % (256 * unit) == 0   # a full tile starts on the tile-size grid
            seq, words = _decode(fo, v, n)
            assert sorted(seq) == list(range(n))
            chans = set(chan[s_:s_ + ln].tolist())
            if key == "fused_ring":
                # block k of a channel folds its order from position k on
                assert words is None
                ks = set(kidx[s_:s_ + ln].tolist())
                assert len(ks) == 1, (s_, ln)
                k = ks.pop()
                for c in chans:
                    order = topo.channels[c].order
                    assert seq == [order[(k + j) % n] for j in range(n)], (c, k)
            else:
                for c in chans:
                    if (v, c) not in checked:
                        checked.add((v, c))
                        want = _oracle_tree_fold(topo.channels[c], xs, dtype)
                        assert _bits(_fold(seq, words, xs, dtype)) == _bits(want), (v, c)


@pytest.mark.parametrize("n,m,nch,chunk,esz,count,pattern,seed", ALL)
def test_stepwise_ring_tasks(dump, n, m, nch, chunk, esz, count, pattern, seed):
    d = _dump(dump, n, m, nch, chunk, esz, count, pattern, seed)
    unit = 16 // esz
    topo = _topo(n, m, nch, pattern, seed)
    slice_ = d["ring_slice"]
    blocks = [(o, b, c) for o, b, c in d["ring_blocks"]]
    want, loop_chan = [], []
    for c, (off, ln) in enumerate(P.channel_ranges(count, unit, nch)):
        for bl in P.ring_loops(off, ln, n, chunk // esz, unit):
            want.extend(bl)
            loop_chan.append(c)
    assert [(o, b) for o, b, _ in blocks] == want
    assert all(c == o // slice_ for o, _, c in blocks)
    # every element of every block lies in exactly one (loop, slice) task cell
    nloops = len(blocks) // n if n else 0
    orders = d["ring_orders"]
    per_loop = {}
    for lp, q, ring, ns in d["ring_tasks"]:
        per_loop.setdefault(lp, []).append((q, ns))
        # the task's ring order is its channel's
        assert orders[ring * 64: ring * 64 + n] == topo.channels[loop_chan[lp]].order
    assert sorted(per_loop) == list(range(nloops))
    for lp, qns in per_loop.items():
        qs = [q for q, _ in qns]
        assert qs == list(range(len(qs)))
        # every task carries its loop's task count (the modulus of the all-reduce's slice skew)
        assert all(ns == len(qs) for _, ns in qns)
        for k in range(n):
            o, b, c = blocks[lp * n + k]
            covered = 0
            for q in qs:
                lo, hi = (c + q) * slice_, (c + q + 1) * slice_
                covered += max(0, min(hi, o + b) - max(lo, o))
            assert covered == b


@pytest.mark.parametrize("n,m,nch,chunk,esz,count,pattern,seed", ALL)
def test_stepwise_tree_tasks_and_records(dump, n, m, nch, chunk, esz, count, pattern, seed):
    d = _dump(dump, n, m, nch, chunk, esz, count, pattern, seed)
    unit = 16 // esz
    topo = _topo(n, m, nch, pattern, seed)
    tasks = d["tree_tasks"]
    _covers([(s_, ln) for s_, ln, _ in tasks], count)
    chan_of = np.full(count, -1, dtype=np.int64)
    for c, (off, ln) in enumerate(P.channel_ranges(count, unit, nch)):
        chan_of[off:off + ln] = c

    def records(c):
        ch = topo.channels[c]
        return tuple(ch.up), tuple(map(tuple, ch.down))
    for s_, ln, c in tasks:
        # every element of a task uses the task channel's tree records
        assert {records(x) for x in set(chan_of[s_:s_ + ln].tolist())} == {records(c)}
    nodes = d["tree_nodes"]
    for c in range(nch):
        ch = topo.channels[c]
        for r in range(n):
            up, d0, d1, d2, depth = nodes[c * n + r]
            assert (up, [d0, d1, d2]) == (ch.up[r], ch.down[r])
            x, dd = r, 0
            while ch.up[x] != -1:
                x, dd = ch.up[x], dd + 1
            assert depth == dd


@pytest.mark.parametrize("n,m,nch,chunk,esz,count,pattern,seed", ALL)
def test_tree_programs_equal_the_oracle_fold(dump, n, m, nch, chunk, esz, count, pattern, seed):
    d = _dump(dump, n, m, nch, chunk, esz, count, pattern, seed)
    topo = _topo(n, m, nch, pattern, seed)
    dtype, xs = _inputs(n, esz, n * 100 + m)
    for prog in d["programs"]:
        assert prog["error"] == 0
        assert prog["nregs"] <= 8
        assert sorted(prog["perm"]) == list(range(n))
        ch = topo.channels[prog["channel"]]
        assert _bits(_run_program(prog, xs, dtype, "sum")) == _bits(_oracle_tree_fold(ch, xs, dtype))
        if all(len(ch.children(r)) <= 1 for r in range(n)):
            assert prog["pure"] == 1   # a chain is a plain fold


@pytest.mark.parametrize("n,m,nch,chunk,esz,count,pattern,seed", ALL)
def test_collective_tiles_follow_the_oracle(dump, n, m, nch, chunk, esz, count, pattern, seed):
    # Reduce-scatter: tile elements of block r fold channel c's ring order
    # from the position after r's; all-gather: tile elements of block k come
    # from rank k.  Tiles cover the N blocks exactly.
    d = _dump(dump, n, m, nch, chunk, esz, count, pattern, seed)
    unit = 16 // esz
    topo = _topo(n, m, nch, pattern, seed)
    block = d["coll_block"]
    assert block == count // unit * unit
    chan = np.full(block, -1, dtype=np.int64)
    for c, (off, ln) in enumerate(P.channel_ranges(block, unit, nch)):
        chan[off:off + ln] = c
    for key in ("fused_rs", "fused_ag"):
        fo = d[key]
        _covers([(s_, ln) for s_, ln, _ in fo["tiles"]], n * block)
        for s_, ln, v in fo["tiles"]:
            owner = v >> 16
            assert s_ // block == owner and (s_ + ln - 1) // block == owner
            if key == "fused_ag":
                continue
            seq, words = _decode(fo, v & 0xFFFF, n)
            assert words is None
            for c in set(chan[s_ - owner * block: s_ - owner * block + ln].tolist()):
                order = topo.channels[c].order
                p = order.index(owner)
                assert seq == [order[(p + 1 + j) % n] for j in range(n)], (owner, c)


@pytest.mark.parametrize("n,m,nch,chunk,esz,count,pattern,seed", ALL)
def test_stepwise_collective_tasks(dump, n, m, nch, chunk, esz, count, pattern, seed):
    # Per channel range of a block and chunk piece: one loop whose step
    # block k is data block order[k-1] at that piece; tasks cover each block.
    d = _dump(dump, n, m, nch, chunk, esz, count, pattern, seed)
    unit = 16 // esz
    topo = _topo(n, m, nch, pattern, seed)
    block, slice_ = d["coll_block"], d["ring_slice"]
    want, loop_chan = [], []
    for c, (off, ln) in enumerate(P.channel_ranges(block, unit, nch)):
        order = topo.channels[c].order
        for o, piece in P.tree_chunks(off, ln, chunk // esz):
            want.extend((order[(k - 1) % n] * block + o, piece) for k in range(n))
            loop_chan.append(c)
    blocks = d["coll_blocks"]
    assert [(o, b) for o, b, _ in blocks] == want
    assert all(c == o // slice_ for o, _, c in blocks)
    orders = d["coll_orders"]
    per_loop = {}
    for lp, q, ring in d["coll_tasks"]:
        per_loop.setdefault(lp, []).append(q)
        assert orders[ring * 64: ring * 64 + n] == topo.channels[loop_chan[lp]].order
    assert sorted(per_loop) == list(range(len(loop_chan)))
    for lp, qs in per_loop.items():
        assert qs == list(range(len(qs)))
        for k in range(n):
            o, b, c = blocks[lp * n + k]
            covered = sum(max(0, min((c + q + 1) * slice_, o + b) - max((c + q) * slice_, o)) for q in qs)
            assert covered == b


def test_rejected_graphs(dump):
    assert dump(4, 4, 2, 64, 4, 10, 1, None) == {"error": 1}            # split needs two ranks per node
    assert dump(4, 2, 1, 64, 4, 10, 0, [[0, 2, 1, 3]]) == {"error": 1}  # rank 2 is not on node 0
    assert dump(4, 1, 1, 64, 4, 10, 0, [[0, 1, 1, 3]]) == {"error": 1}  # rank 1 twice
    assert dump(4, 1, 1, 64, 4, 10, 3, None) == {"error": 1}            # unknown pattern
