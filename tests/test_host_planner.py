"""Host planner checks (CPU only): the library's tiles, stepwise tasks and
compiled tree programs, dumped by a small C++ driver built from the
host-only planner sources with AddressSanitizer and UndefinedBehavior-
Sanitizer, are compared with the oracle's partition and tree folds."""

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


@pytest.fixture(scope="module")
def dump():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    os.makedirs(BUILD, exist_ok=True)
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I" + CSRC, os.path.join(ROOT, "tests", "host", "planner_dump.cpp"),
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "topology.cpp"), "-o", EXE]
    subprocess.run(cmd, check=True, capture_output=True)

    def run(n, m, nch, chunk_bytes, esz, count):
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1")
        out = subprocess.run([EXE, str(n), str(m), str(nch), str(chunk_bytes), str(esz), str(count)],
                             check=True, capture_output=True, text=True, env=env)
        return json.loads(out.stdout)
    return run


CASES = [(4, 1, 1, 512 * 1024, 4, 1024), (8, 1, 12, 4096, 4, 37 * 1024 + 5), (16, 16, 8, 1024, 2, 20000),
         (15, 15, 8, 1024, 2, 20003), (32, 4, 16, 2048, 2, 30001), (32, 4, 16, 2048, 8, 9000),
         (6, 3, 5, 64, 8, 1025), (3, 3, 2, 16, 4, 257), (1, 1, 1, 64, 4, 100), (64, 8, 64, 256, 4, 6157),
         (2, 2, 3, 64, 2, 7), (12, 3, 4, 512, 4, 0), (5, 5, 7, 48, 4, 9)]


def _covers(pieces, count):
    pos = 0
    for start, n in pieces:
        assert start == pos and n > 0, (start, n, pos)
        pos += n
    assert pos == count


@pytest.mark.parametrize("n,m,nch,chunk,esz,count", CASES)
def test_fused_tiles_follow_the_partition(dump, n, m, nch, chunk, esz, count):
    d = dump(n, m, nch, chunk, esz, count)
    unit = 16 // esz
    topo = T.build_topology(n, m, nch)
    # expected variant per element: ring -> rank-chunk index, tree -> tree index
    ring_var = np.full(count, -1, dtype=np.int64)
    tree_var = np.full(count, -1, dtype=np.int64)
    for c, (off, ln) in enumerate(P.channel_ranges(count, unit, nch)):
        tree_var[off:off + ln] = topo.channels[c].tree_index
        for blocks in P.ring_loops(off, ln, n, chunk // esz, unit):
            for k, (o, b) in enumerate(blocks):
                ring_var[o:o + b] = k
    for key, want in (("tiles_ring", ring_var), ("tiles_tree", tree_var)):
        tiles = d[key]
        _covers([(s, ln) for s, ln, _ in tiles], count)
        for s, ln, v in tiles:
            assert (want[s:s + ln] == v).all(), (key, s, ln, v)
            assert ln <= 256 * unit
            # a full tile starts on the tile-size grid
            if ln == 256 * unit:
                assert s % (256 * unit) == 0


@pytest.mark.parametrize("n,m,nch,chunk,esz,count", CASES)
def test_stepwise_ring_tasks(dump, n, m, nch, chunk, esz, count):
    d = dump(n, m, nch, chunk, esz, count)
    unit = 16 // esz
    slice_ = d["ring_slice"]
    blocks = [(o, b, c) for o, b, c in d["ring_blocks"]]
    want = []
    for off, ln in P.channel_ranges(count, unit, nch):
        for bl in P.ring_loops(off, ln, n, chunk // esz, unit):
            want.extend(bl)
    assert [(o, b) for o, b, _ in blocks] == want
    assert all(c == o // slice_ for o, _, c in blocks)
    # every element of every block lies in exactly one (loop, slice) task cell
    nloops = len(blocks) // n if n else 0
    tasks = d["ring_tasks"]
    per_loop = {}
    for lp, q in tasks:
        per_loop.setdefault(lp, []).append(q)
    assert sorted(per_loop) == list(range(nloops))
    for lp, qs in per_loop.items():
        assert qs == list(range(len(qs)))
        for k in range(n):
            o, b, c = blocks[lp * n + k]
            covered = 0
            for q in qs:
                lo, hi = (c + q) * slice_, (c + q + 1) * slice_
                covered += max(0, min(hi, o + b) - max(lo, o))
            assert covered == b


@pytest.mark.parametrize("n,m,nch,chunk,esz,count", CASES)
def test_stepwise_tree_tasks_and_records(dump, n, m, nch, chunk, esz, count):
    d = dump(n, m, nch, chunk, esz, count)
    unit = 16 // esz
    topo = T.build_topology(n, m, nch)
    tasks = d["tree_tasks"]
    _covers([(s, ln) for s, ln, _ in tasks], count)
    chan_of = np.full(count, -1, dtype=np.int64)
    for c, (off, ln) in enumerate(P.channel_ranges(count, unit, nch)):
        chan_of[off:off + ln] = c
    for s, ln, c in tasks:
        # every element of a task uses the task's node-level tree
        trees = {topo.channels[x].tree_index for x in set(chan_of[s:s + ln].tolist())}
        assert trees == {topo.channels[c].tree_index}
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


def _run_program(prog, xs, dtype, op):
    """Evaluate a compiled register program on the oracle's arithmetic."""
    regs = [None] * 8
    for j, (rank, w) in enumerate(zip(prog["perm"], prog["instr"])):
        dreg = (w >> 1) & 7
        regs[dreg] = N.combine(dtype, op, regs[dreg], xs[rank]) if w & 1 else xs[rank].copy()
        for p_ in range(1, (w >> 4) + 1):
            regs[dreg - p_] = N.combine(dtype, op, regs[dreg - p_], regs[dreg - p_ + 1])
    return regs[0]


@pytest.mark.parametrize("n,m,nch,chunk,esz,count", [c for c in CASES if c[0] > 0])
def test_tree_programs_equal_the_oracle_fold(dump, n, m, nch, chunk, esz, count):
    d = dump(n, m, nch, chunk, esz, count)
    topo = T.build_topology(n, m, nch)
    rng = np.random.default_rng(n * 100 + m)
    dtype = {2: "bf16", 4: "f32", 8: "i64"}[esz]
    xs = [rng.standard_normal(64).astype(np.float32) for _ in range(n)]
    if dtype == "bf16":
        xs = [N.f32_to_bf16(x) for x in xs]
    elif dtype == "i64":
        xs = [rng.integers(-1 << 40, 1 << 40, size=64) for _ in range(n)]
    for prog in d["programs"]:
        assert prog["error"] == 0
        assert prog["nregs"] <= 8
        assert sorted(prog["perm"]) == list(range(n))
        ch = next(c for c in topo.channels if c.tree_index == prog["tree"])
        want = TR.tree_allreduce_chunk(xs, ch.up, ch.down, lambda a, b: N.combine(dtype, "sum", a, b),
                                       lambda a: a.copy())[0]
        got = _run_program(prog, xs, dtype, "sum")
        assert np.array_equal(np.asarray(got).view(np.uint8), np.asarray(want).view(np.uint8))
        if m == 1:
            assert prog["pure"] == 1   # a chain is a plain fold
