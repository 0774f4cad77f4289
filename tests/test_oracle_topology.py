"""Pins of the oracle topology (CPU only).

Each test checks the oracle against something the pages print or that the
mathematics fixes, not against a retyped copy of the oracle."""

import pytest

from oracle import topology as T
from tests.conftest import golden_lines


def test_probe_table_roots_depths_overlap():
    # "NCCL 专家课程 13", section "直接执行源码中的 DTree".
    for line in golden_lines("dtree_probe_table.txt"):
        n, kind, r0, r1, d0, d1, overlap = line.split()
        n = int(n)
        assert T.node_tree_root(n, 0) == int(r0)
        assert T.node_tree_root(n, 1) == int(r1)
        assert T.node_tree_depth(n, 0) == int(d0)
        assert T.node_tree_depth(n, 1) == int(d1)
        shared = T.interior_nodes(n, 0) & T.interior_nodes(n, 1)
        want = set() if overlap == "none" else {int(x) for x in overlap.split(",")}
        assert shared == want, (n, shared)
        if kind == "mirror":
            assert n % 2 == 0
        elif kind == "shift":
            assert n % 2 == 1


def test_four_node_trees_match_drawings():
    # Sections "Btree 的 bit 构造" and "双树：偶数 mirror，奇数 shift".
    for line in golden_lines("dtree4_trees.txt"):
        parts = line.split()
        if parts[0] == "INTERIOR":
            which = int(parts[1])
            assert T.interior_nodes(4, which) == {int(x) for x in parts[2].split(",")}
            continue
        which, node, parent, children = int(parts[0]), int(parts[1]), int(parts[2]), parts[3]
        p, c0, c1, _ = T.dtree(4, node)[which]
        assert p == parent
        got = [c for c in (c0, c1) if c != -1]
        want = [] if children == "none" else [int(c) for c in children.split(",")]
        assert got == want, (which, node, got, want)


def test_chain_roles_and_depth():
    # "NCCL 专家课程 13", sections "每种 rank 的操作" and "节点间连接".
    topo = T.build_topology(4, 1, 1)
    ch = topo.channels[0]
    for line in golden_lines("chain4_roles.txt"):
        parts = line.split()
        if parts[0] == "DEPTH":
            assert ch.depth == int(parts[1])
            assert ch.true_depth() == int(parts[1])
            continue
        r, role, parent, child = int(parts[0]), parts[1], int(parts[2]), int(parts[3])
        assert ch.up[r] == parent
        assert ch.down[r][0] == child
        assert ch.down[r][1:] == [-1, -1]
        is_root = ch.up[r] == -1
        is_leaf = ch.down[r][0] == -1
        assert role == ("root" if is_root else "leaf" if is_leaf else "internal")


def test_btree_special_cases():
    # Closed forms: a single node is a lone root; two nodes are 0 -> 1.
    assert T.btree(1, 0) == (-1, -1, -1, None)
    assert T.btree(2, 0)[:3] == (-1, -1, 1)
    assert T.btree(2, 1)[:3] == (0, -1, -1)
    # For n a power of two, node n/2 is node 0's only child and every odd node
    # is a leaf (its lowest set bit is 1, so it has no lower half-step).
    for n in (4, 8, 16, 32, 64):
        assert T.btree(n, 0)[2] == n // 2
        for r in range(1, n, 2):
            assert T.btree(n, r)[1:3] == (-1, -1)


@pytest.mark.parametrize("n", range(1, 70))
def test_node_trees_are_trees_of_log_depth(n):
    # Invariants: both node-level trees are valid trees over 0..n-1 with at
    # most two children per node, the root with at most one, and depth at
    # most ceil(log2 n) (the bit construction halves the offset per level).
    for which in (0, 1):
        parents = [T.dtree(n, m)[which][0] for m in range(n)]
        kids = {m: [c for c in T.dtree(n, m)[which][1:3] if c != -1] for m in range(n)}
        assert parents.count(-1) == 1
        root = parents.index(-1)
        assert len(kids[root]) <= 1
        for m in range(n):
            for c in kids[m]:
                assert parents[c] == m
        assert sum(len(k) for k in kids.values()) == n - 1
        depth = T.node_tree_depth(n, which)
        bound = 0 if n == 1 else (n - 1).bit_length()
        assert depth <= bound
    if n % 2 == 0:
        # Mirror: tree 1 is tree 0 relabelled m -> n-1-m.
        for m in range(n):
            p0 = T.dtree(n, m)[0][0]
            p1 = T.dtree(n, n - 1 - m)[1][0]
            assert p1 == (-1 if p0 == -1 else n - 1 - p0)
        assert not (T.interior_nodes(n, 0) & T.interior_nodes(n, 1))
    else:
        # Shift: tree 1 is tree 0 relabelled m -> m+1 mod n.
        for m in range(n):
            p0 = T.dtree(n, m)[0][0]
            p1 = T.dtree(n, (m + 1) % n)[1][0]
            assert p1 == (-1 if p0 == -1 else (p0 + 1) % n)


def _shapes():
    for n in range(1, 65):
        for m in range(1, n + 1):
            if n % m == 0 and (n <= 16 or m in (1, 2, n // 8 if n % 8 == 0 else 1, n)):
                yield n, m


def test_hierarchical_graph_assertions_all_shapes():
    # "NCCL 专家课程 13", section "从 GRAPH 日志复原 active tree": parent/child
    # symmetry, one root, N-1 edges, acyclic, all reach the root; arity bounds
    # of section "数据结构不是纯二叉树".
    count = 0
    for n, m in _shapes():
        for nch in (1, 2, 3, 8):
            topo = T.build_topology(n, m, nch)
            for c, ch in enumerate(topo.channels):
                T.check_tree(ch)
                assert ch.tree_index == (0 if c < (nch + 1) // 2 else 1)
                count += 1
    assert count > 500


def test_single_node_is_a_chain():
    # Section "可证伪预测" item 2 and the active-tree table of section "本机真实
    # 树形": on one node every channel's tree has fan-out 1 and depth N-1.
    for n in range(1, 33):
        for ch in T.build_topology(n, 1, 4).channels:
            assert max(len(ch.children(r)) for r in range(n)) <= 1
            assert ch.true_depth() == n - 1
            assert ch.root == 0


def test_depth_formula_where_exact():
    # Section "节点间连接": depth = L - 1 + floor(log2 M), an approximation.
    # It is exact for a chain and for power-of-two node counts with a chain
    # below every head; for 15 nodes the true depth exceeds it by one.
    for n, m in ((4, 1), (8, 1), (32, 4), (16, 16), (64, 8)):
        topo = T.build_topology(n, m, 2)
        for ch in topo.channels:
            assert ch.true_depth() == ch.depth == n // m - 1 + T.log2i(m)
    topo = T.build_topology(15, 15, 2)
    assert topo.channels[0].depth == 3
    assert topo.channels[0].true_depth() == 4


def test_hierarchical_heads_and_slots():
    # Heads are local index 0; a head keeps its chain child in slot 0 and
    # takes node-level children in the next free slots, child0 before child1.
    topo = T.build_topology(32, 4, 2)
    ch0, ch1 = topo.channels
    # tree 0 over 4 nodes: 0 -> 2 -> {1, 3}; heads are ranks 0, 8, 16, 24.
    assert ch0.up[0] == -1 and ch0.down[0] == [1, 16, -1]
    assert ch0.up[16] == 0 and ch0.down[16] == [17, 8, 24]
    assert ch0.up[8] == 16 and ch0.up[24] == 16
    # tree 1: 3 -> 1 -> {2, 0}
    assert ch1.up[24] == -1 and ch1.down[24] == [25, 8, -1]
    assert ch1.down[8] == [9, 16, 0]
    # non-head ranks are pure chain members in both channels
    for ch in (ch0, ch1):
        assert ch.up[5] == 4 and ch.down[5] == [6, -1, -1]
        assert ch.down[31] == [-1, -1, -1]


def test_slot_overflow_is_an_error():
    down = [[1, 2, 3]]
    with pytest.raises(T.TopologyError):
        T._attach_down(down, 0, 4)


def test_step_counts_figure():
    # Figure 2 of the interview page: ring 2(n-1) steps; a balanced tree
    # about 2*log2(n) (levels up plus levels down).  The node-level tree of
    # the double tree is that balanced tree.
    for line in golden_lines("step_counts.txt"):
        n, ring_steps, tree_steps = (int(x) for x in line.split())
        assert 2 * (n - 1) == ring_steps
        assert 2 * T.node_tree_depth(n, 0) == tree_steps


# ---------------------------------------------------------------------------
# Per-channel chain orders and head patterns.

def _chain_walk(ch):
    """Root-to-leaf walk along first children (a chain has one path)."""
    out, x = [], ch.root
    while x != -1:
        out.append(x)
        kids = ch.children(x)
        x = kids[0] if kids else -1
    return out


def test_v100_channel_chains_table():
    # "NCCL 专家课程 13", section "从 GRAPH 日志复原 active tree": 12 channels per
    # world size, each a chain in its own order; 108 records in all.
    rows = [ln.split() for ln in golden_lines("v100_channel_chains.txt") if ln.startswith("CHAINS")]
    records = int(next(ln.split()[1] for ln in golden_lines("v100_channel_chains.txt")
                       if ln.startswith("RECORDS")))
    total = 0
    for n in (2, 3, 4):
        intra = [None] * 12
        want = {}
        for _, world, chans, order, depth, fan in rows:
            if int(world) != n:
                continue
            order = [int(x) for x in order.split("-")]
            for c in map(int, chans.split(",")):
                intra[c] = order
                want[c] = (order, int(depth), int(fan))
        assert all(o is not None for o in intra), n
        topo = T.build_topology(n, 1, 12, intra=intra)
        for c, ch in enumerate(topo.channels):
            T.check_tree(ch)
            order, depth, fan = want[c]
            assert ch.root == order[0]
            assert _chain_walk(ch) == order
            assert ch.true_depth() == depth
            assert max(len(ch.children(r)) for r in range(n)) == fan
            total += n
        distinct = {tuple(_chain_walk(ch)) for ch in topo.channels}
        assert len(distinct) == {2: 2, 3: 2, 4: 3}[n]
    assert total == records


def test_head_patterns_hand_worked_3x2():
    intra = [1, 0, 2, 3, 5, 4]
    got = {}
    for pattern in T.PATTERNS:
        topo = T.build_topology(6, 3, 2, pattern, [intra, intra])
        assert [ch.tree_index for ch in topo.channels] == [0, 1]
        for ch in topo.channels:
            T.check_tree(ch)
            got[(pattern, ch.tree_index)] = (ch.up, ch.down)
    seen = 0
    for line in golden_lines("head_patterns_3x2.txt"):
        left, right = line.split("|")
        pattern, tree, _, *ups = left.split()
        downs = [[int(v) for v in d.split(",")] for d in right.split()[1:]]
        assert got[(pattern, int(tree))] == ([int(u) for u in ups], downs), (pattern, tree)
        seen += 1
    assert seen == 6


def _random_orders(rng, n, m, nch):
    L = n // m
    out = []
    for _ in range(nch):
        row = []
        for node in range(m):
            row += [int(x) for x in rng.permutation(range(node * L, (node + 1) * L))]
        out.append(row)
    return out


@pytest.mark.parametrize("pattern", ["tree", "split", "balanced"])
@pytest.mark.parametrize("n,m", [(4, 2), (6, 3), (8, 2), (8, 4), (12, 4), (16, 2), (16, 8), (24, 3),
                                 (32, 4), (30, 5), (64, 8), (64, 32), (18, 9), (10, 5), (14, 7)])
def test_pattern_invariants_random_orders(pattern, n, m):
    # Contracting every node to one vertex gives the node-level tree of the
    # channel; inside a node the edges are the chain in the channel's order;
    # the edge to the parent node leaves from chain position 0 and lands on
    # the parent node's child0 or child1 head.
    import numpy as np
    rng = np.random.default_rng(n * 1000 + m)
    L = n // m
    pos_p, pos_c0, pos_c1 = T.head_positions(pattern)
    nch = 4
    intra = _random_orders(rng, n, m, nch)
    topo = T.build_topology(n, m, nch, pattern, intra)
    for c, ch in enumerate(topo.channels):
        T.check_tree(ch)
        assert ch.order == intra[c]
        chains = [intra[c][k * L:(k + 1) * L] for k in range(m)]
        pos = {r: (k, chains[k].index(r)) for k in range(m) for r in chains[k]}
        for r in range(n):
            k, i = pos[r]
            u = ch.up[r]
            node_parent = T.dtree(m, k)[ch.tree_index][0]
            if i > 0:
                assert u == chains[k][i - 1]
            elif node_parent == -1:
                assert u == -1
            else:
                ctype = T.dtree(m, k)[ch.tree_index][3]
                kp, ip = pos[u]
                assert kp == node_parent
                assert ip == (pos_c0 if ctype == 0 else pos_c1)
            # children: the chain successor first, then the child nodes' heads
            kids = ch.children(r)
            want = [chains[k][i + 1]] if i < L - 1 else []
            _, c0, c1, _ = T.dtree(m, k)[ch.tree_index]
            if c0 != -1 and i == pos_c0:
                want.append(chains[c0][pos_p])
            if c1 != -1 and i == pos_c1:
                want.append(chains[c1][pos_p])
            assert kids == want, (c, r)


def test_pattern_needs_two_ranks_per_node_and_valid_orders():
    with pytest.raises(ValueError):
        T.build_topology(4, 4, 2, "split")
    with pytest.raises(ValueError):
        T.build_topology(4, 4, 2, "balanced")
    T.build_topology(4, 4, 2, "tree")
    with pytest.raises(ValueError):
        T.build_topology(4, 2, 1, "tree", [[0, 2, 1, 3]])   # rank 2 is not on node 0
    with pytest.raises(ValueError):
        T.build_topology(4, 1, 2, "tree", [[0, 1, 2, 3]])   # one order per channel
    with pytest.raises(ValueError):
        T.build_topology(4, 1, 1, "ring", None)


def test_identity_orders_match_the_default():
    for n, m in ((8, 1), (16, 16), (32, 4), (6, 3)):
        a = T.build_topology(n, m, 4)
        b = T.build_topology(n, m, 4, "tree", [list(range(n))] * 4)
        assert [(c.up, c.down) for c in a.channels] == [(c.up, c.down) for c in b.channels]
