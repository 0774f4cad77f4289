"""Pins of the oracle ring and tree simulators (CPU only)."""

import numpy as np
import pytest

from oracle import allreduce as A
from oracle import ring as R
from oracle import topology as T
from oracle import tree as TR
from tests.conftest import golden_lines


def _sym_ring(n):
    letters = "abcdefghijklmnop"[:n]
    bufs = [[frozenset(letters[r]) for _ in range(n)] for r in range(n)]
    trace = []
    sent = [0] * n
    R.ring_allreduce_blocks(bufs, lambda a, b: a | b, lambda a: a, trace=trace, sent=sent,
                            size=lambda a: 1)
    return bufs, trace, sent


def test_ring_four_rank_step_table():
    # Interview page, Figure 1: every intermediate state of all 4 ranks.
    _, trace, sent = _sym_ring(4)
    states = {f"{ph}{s}": rows for (ph, s), rows in trace}
    for line in golden_lines("ring4_step_table.txt"):
        parts = line.split()
        if parts[0] == "SENT_BLOCKS_PER_RANK":
            assert sent == [int(parts[1])] * 4
            continue
        label, gpu, blocks = parts[0], int(parts[1][3:]), parts[2:]
        got = ["".join(sorted(b)) for b in states[label][gpu]]
        assert got == blocks, (label, gpu, got, blocks)


def test_ring_symbolic_any_n_ends_full_and_sends_2n_minus_2():
    # After reduce-scatter rank r holds the full block (r+1) mod n; after
    # all-gather every block everywhere is full; each rank sends 2(n-1)
    # blocks (interview page, section "推导 / 关键公式").
    for n in range(1, 12):
        bufs, trace, sent = _sym_ring(n)
        full = frozenset("abcdefghijklmnop"[:n])
        assert all(b == full for row in bufs for b in row)
        assert sent == [2 * (n - 1)] * n
        if n > 1:
            after_rs = trace[n - 2][1]
            for r in range(n):
                assert after_rs[r][(r + 1) % n] == full


def test_two_rank_example_ring_and_tree():
    # Interview page, section "先弄清楚:每个概念是什么".
    rows = [ln.split("->") for ln in golden_lines("allreduce_2rank_example.txt")]
    inputs = [np.array([int(v) for v in lhs.split(":")[1].split()], dtype=np.int32) for lhs, _ in rows]
    want = [[int(v) for v in rhs.split()] for _, rhs in rows]
    for algo, nnodes in (("ring", 1), ("tree", 1), ("tree", 2)):
        out = A.allreduce(inputs, nnodes, algo, 1, 16, "i32", "sum")
        assert [o.tolist() for o in out] == want, (algo, nnodes)


@pytest.mark.parametrize("n,count", [(2, 7), (3, 10), (4, 1024), (5, 101), (8, 999), (9, 64)])
def test_ring_with_unit_one_is_the_per_block_left_fold(n, count):
    # Interview page, section "手撕代码": each rank's vector is cut into n parts
    # the numpy.array_split way, and part k is reduced along the ring starting
    # at rank k.  With a unit of one element, one channel and one loop, the
    # oracle's step simulation must equal that closed form element by
    # element: acc = x_k; acc = rnd(acc + x_{k+j mod n}) for j = 1 .. n-1,
    # every add a plain IEEE single add (numpy float32 scalars).
    rng = np.random.default_rng(100 + n)
    xs = [rng.standard_normal(count).astype(np.float32) for _ in range(n)]
    out = A.allreduce(xs, 1, "ring", 1, 4 * count, "f32", "sum", unit_bytes=4)
    parts = np.array_split(np.arange(count), n)
    want = np.empty(count, dtype=np.float32)
    for k, idx in enumerate(parts):
        for i in idx:
            acc = np.float32(xs[k][i])
            for j in range(1, n):
                acc = np.float32(acc + xs[(k + j) % n][i])
            want[i] = acc
    for o in out:
        assert np.array_equal(o.view(np.uint32), want.view(np.uint32))


def _order_pin(tag):
    vals = {}
    for line in golden_lines("order_pins_f32.txt"):
        name, kind, *nums = line.split()
        if name == tag:
            vals[kind] = [float(x) for x in nums]
    return vals


def test_ring_fold_order_pin():
    pin = _order_pin("RING3")
    inputs = [np.full(12, v, dtype=np.float32) for v in pin["inputs"]]
    out = A.allreduce(inputs, 1, "ring", 1, 512 * 1024, "f32", "sum")
    for o in out:
        assert o.tolist() == pin["expect"]


def test_chain_fold_order_pin():
    pin = _order_pin("CHAIN4")
    inputs = [np.full(4, v, dtype=np.float32) for v in pin["inputs"]]
    out = A.allreduce(inputs, 1, "tree", 1, 512 * 1024, "f32", "sum")
    for o in out:
        assert o.tolist() == pin["expect"]


def test_permuted_ring_fold_order_pin():
    pin = _order_pin("RING3P")
    order = [int(x) for x in pin["order"]]
    inputs = [np.full(12, v, dtype=np.float32) for v in pin["inputs"]]
    out = A.allreduce(inputs, 1, "ring", 1, 512 * 1024, "f32", "sum", intra=[order])
    for o in out:
        assert o.tolist() == pin["expect"]
    # the sampled form agrees
    at = A.allreduce_at(inputs, np.arange(12), 1, "ring", 1, 512 * 1024, "f32", "sum", intra=[order])
    assert at.tolist() == pin["expect"]


def test_permuted_chain_fold_order_pin():
    pin = _order_pin("CHAIN4P")
    order = [int(x) for x in pin["order"]]
    inputs = [np.full(4, v, dtype=np.float32) for v in pin["inputs"]]
    out = A.allreduce(inputs, 1, "tree", 1, 512 * 1024, "f32", "sum", intra=[order])
    for o in out:
        assert o.tolist() == pin["expect"]


@pytest.mark.parametrize("pattern", ["tree", "split", "balanced"])
def test_head_pattern_fold_order_pin(pattern):
    pin = _order_pin("HEADS4")
    inputs = [np.full(4, v, dtype=np.float32) for v in pin["inputs"]]
    out = A.allreduce(inputs, 2, "tree", 1, 512 * 1024, "f32", "sum", pattern=pattern)
    for o in out:
        assert o.tolist() == pin["expect_" + pattern]
    at = A.allreduce_at(inputs, np.arange(4), 2, "tree", 1, 512 * 1024, "f32", "sum", pattern=pattern)
    assert at.tolist() == pin["expect_" + pattern]


def test_ring_order_sends_per_rank():
    # A permuted ring moves the same volume: every rank sends 2(N-1) blocks.
    n, count = 4, 64
    inputs = [np.zeros(count, dtype=np.int32) for _ in range(n)]
    stats = {}
    A.allreduce(inputs, 1, "ring", 1, 16 * 1024, "i32", "sum", stats=stats, intra=[[2, 0, 3, 1]])
    assert stats["sent_elems"] == [2 * (n - 1) * count // n] * n


def test_tree_symbolic_every_shape_reaches_everyone():
    # Reduce-up collects every rank exactly once at the root; broadcast-down
    # hands the same result to every rank.  Sets would hide a double count,
    # so count contributions with multisets (sorted tuples).
    for n, m in ((1, 1), (2, 2), (3, 3), (4, 1), (8, 2), (15, 15), (16, 16), (32, 4), (24, 3)):
        topo = T.build_topology(n, m, 2)
        for ch in topo.channels:
            out = TR.tree_allreduce_chunk([(r,) for r in range(n)], ch.up, ch.down,
                                          lambda a, b: tuple(sorted(a + b)), lambda a: a)
            assert all(o == tuple(range(n)) for o in out)


def _volume(n, nnodes, algo, nch, count, dtype="i32"):
    inputs = [np.zeros(count, dtype=np.int32) for _ in range(n)]
    stats = {}
    A.allreduce(inputs, nnodes, algo, nch, 4 * count, dtype, "sum", stats=stats)
    return stats["sent_elems"]


def test_send_volume_ring():
    # Interview page, Figure 1 caption and section "推导 / 关键公式": each rank
    # sends 2(n-1) blocks of S/n.
    for n in (2, 3, 4, 5, 8):
        count = 4 * n * 16
        sent = _volume(n, 1, "ring", 1, count)
        assert sent == [2 * (n - 1) * count // n] * n


def test_send_volume_tree_chain_and_double_tree():
    # Every tree edge carries the data once up and once down, so the total
    # is 2(N-1)S whether one tree or two carry the message (course page,
    # section "为什么不是发送两份完整消息"); on a chain the ends send S and the
    # middle ranks 2S; with the even-n double tree no rank sends more than 2S
    # (interview page, the tree row of the comparison table).
    count = 1024
    for n in (2, 4, 8):
        sent = _volume(n, 1, "tree", 1, count)
        assert sum(sent) == 2 * (n - 1) * count
        assert sent[0] == count and sent[-1] == count
        assert all(s == 2 * count for s in sent[1:-1])
    for n in (4, 8, 16, 32):
        sent = _volume(n, n, "tree", 2, count)
        assert sum(sent) == 2 * (n - 1) * count
        assert max(sent) == 2 * count
    for n in (5, 15):
        sent = _volume(n, n, "tree", 2, count)
        assert sum(sent) == 2 * (n - 1) * count
