"""Oracle: tree topology of the all-reduce data path (test infrastructure only).

Sources (page title, then section):

* "NCCL 专家课程 13：Tree、双树、层次化连接与真实交叉区间" (blog.cptz.space, NCCL
  course chapter 13), sections
  - "先固定方向" and "数据结构不是纯二叉树": a tree record per channel holds a
    parent (``up``, -1 at the root) and three child slots (``down``, -1 when
    empty); the root has at most two children, any other rank at most three.
  - "Btree 的 bit 构造": the node-level binary tree built from bit operations.
  - "双树：偶数 mirror，奇数 shift": the second tree, mirrored for an even node
    count and shifted by one for an odd node count.
  - "节点内先形成链": inside a node the ranks form a chain (parent = previous
    rank, first child = next rank) and the channel records are duplicated
    so that each copy can carry one of the two node-level trees.
  - "节点间连接": node-level edges are attached to each node's head rank; the
    ``depth`` field is the approximation  L - 1 + floor(log2(nnodes)).
  - "从 GRAPH 日志复原 active tree": the structural assertions (parent/child
    symmetry, one root, N-1 edges, no cycle, every rank reaches the root).
  - "直接执行源码中的 DTree": the probe table of roots and depths.

* "NCCL 专家课程 13", section "节点内先形成链" (the preset code): per channel
  the chain follows that channel's intra-node order, and the head pattern
  picks which chain positions carry the node-level edges: the parent edge
  always leaves from position 0; the child edges arrive at position 0 for the
  plain tree pattern, at position 1 for the split pattern, and at position 1
  (child0) and 0 (child1) for the balanced pattern.
* "NCCL代码分析", section "Tree搜索": the three intra-node tree
  patterns (tree, split tree, balanced tree).
* Section "节点间连接" (connectTrees): a node's parent head links up to the
  parent node's child0 head or child1 head, as the node's child type says; a
  node's child0 (child1) head takes the parent head of its child0 (child1)
  node as a child.

Readings where the pages are silent (each listed in the design doc):

* The intra-node order of every channel is given by the caller (the pages
  obtain it from a hardware graph search); by default it is the identity
  (local i = rank node*L + i).  The ring of a channel runs through node 0's
  order, then node 1's, and so on (the ring joins the nodes' channels end to
  end).
* The split and balanced patterns name chain position 1, so they need at
  least two ranks per node.
* Attaching a parent writes ``up``; attaching a child writes the first empty
  ``down`` slot, children taken in the order child0 then child1; a full record
  is an error.
* Of ``nchannels`` channels the first ceil(nchannels/2) use tree 0 and the
  rest tree 1 (the duplicated copies).  With one node both trees are the
  bare chain.

Pins (tests/test_oracle_topology.py): the probe table, the 4-node drawings,
the chain roles, the structural assertions for every shape up to 64 ranks and
the depth formula values that the pages work out, the per-channel chains of
the pages' 4-GPU table, and hand-worked records of the three patterns.
"""

from __future__ import annotations

from dataclasses import dataclass, field


def btree_parent(n: int, r: int) -> int:
    """Parent of node r in the node-level binary tree over 0..n-1 (-1 for
    the root, node 0).  Section "Btree 的 bit 构造": with b the lowest set bit
    of r, the parent is the node one level up, whose lowest set bit is 2b:
    of the two neighbours r - b and r + b that is the one with bit 2b set
    (clear bit b of r, set bit 2b).  When that node does not exist (r + b >=
    n) the parent is r - b (bit b cleared, nothing set)."""
    if not (0 <= r < n):
        raise ValueError(f"rank {r} outside 0..{n - 1}")
    if r == 0:
        return -1
    b = r & -r
    up = r - b if r & (2 * b) else r + b
    return up if up < n else r - b


def btree(n: int, r: int) -> tuple[int, int, int, int | None]:
    """Node r of the node-level binary tree over 0..n-1.

    Returns ``(parent, child0, child1, child_type)``.  The tree is the one
    the parent rule of :func:`btree_parent` defines; the children of r are
    the nodes whose parent r is, at most one below r (child0) and one above
    (child1).  ``child_type`` says whether r lies below (0) or above (1) its
    parent; None at the root.  (Section "Btree 的 bit 构造": node 0 is the
    root with only its second child.)
    """
    parent = btree_parent(n, r)
    below = [x for x in range(n) if x < r and btree_parent(n, x) == r]
    above = [x for x in range(n) if x > r and btree_parent(n, x) == r]
    if len(below) > 1 or len(above) > 1:
        raise TopologyError(f"node {r} of {n} would have more than one child on a side")
    child0 = below[0] if below else -1
    child1 = above[0] if above else -1
    child_type = None if parent == -1 else (0 if r < parent else 1)
    return parent, child0, child1, child_type


def dtree(n: int, r: int):
    """The two node-level trees of node r.

    Tree 0 is :func:`btree`.  Tree 1 is tree 0 with its node ids relabelled
    by sigma: x -> n-1-x (mirror) for even n, x -> x+1 mod n (shift) for odd
    n.  So node r of tree 1 is node sigma^-1(r) of tree 0 with every id it
    names mapped through sigma; the child slots and the child type carry
    over unchanged.  (Section "双树：偶数 mirror，奇数 shift".)
    """
    if n % 2 == 1:
        def sigma(x):
            return (x + 1) % n
        source = (r - 1) % n
    else:
        def sigma(x):
            return n - 1 - x
        source = n - 1 - r
    p, c0, c1, ct = btree(n, source)
    t1 = tuple(-1 if x == -1 else sigma(x) for x in (p, c0, c1)) + (ct,)
    return btree(n, r), t1


def log2i(x: int) -> int:
    """floor(log2(x)) for x >= 1."""
    out = 0
    while x >= 2:
        x >>= 1
        out += 1
    return out


class TopologyError(Exception):
    """A tree record overflowed or a structural assertion failed."""


@dataclass
class ChannelTree:
    """Per-rank tree records of one channel."""
    up: list[int]
    down: list[list[int]]
    tree_index: int            # 0 or 1: which node-level tree this channel uses
    depth: int                 # the pages' approximation, metadata only
    order: list[int] = field(default_factory=list)   # ring / chain order of the ranks

    @property
    def root(self) -> int:
        roots = [r for r, u in enumerate(self.up) if u == -1]
        if len(roots) != 1:
            raise TopologyError(f"expected one root, found {roots}")
        return roots[0]

    def children(self, r: int) -> list[int]:
        return [c for c in self.down[r] if c != -1]

    def true_depth(self) -> int:
        """Longest root-to-leaf path, in edges."""
        best = 0
        for r in range(len(self.up)):
            d, x = 0, r
            while self.up[x] != -1:
                x = self.up[x]
                d += 1
            best = max(best, d)
        return best


@dataclass
class Topology:
    nranks: int
    nnodes: int
    nchannels: int
    channels: list[ChannelTree] = field(default_factory=list)
    pattern: str = "tree"

    @property
    def local_ranks(self) -> int:
        return self.nranks // self.nnodes


def _attach_up(up: list[int], r: int, parent: int) -> None:
    if parent == -1:
        return
    up[r] = parent


def _attach_down(down: list[list[int]], r: int, child: int) -> None:
    if child == -1:
        return
    for slot in range(3):
        if down[r][slot] == -1:
            down[r][slot] = child
            return
    raise TopologyError(f"rank {r} has no free child slot for {child}")


PATTERNS = ("tree", "split", "balanced")


def head_positions(pattern: str) -> tuple[int, int, int]:
    """Chain positions of the (parent, child0, child1) heads of a node
    (section "节点内先形成链")."""
    if pattern == "tree":
        return 0, 0, 0
    if pattern == "split":
        return 0, 1, 1
    if pattern == "balanced":
        return 0, 1, 0
    raise ValueError(f"unknown pattern {pattern!r}")


def _check_intra(intra, nranks: int, nnodes: int, nchannels: int) -> list[list[int]]:
    L = nranks // nnodes
    if intra is None:
        return [list(range(nranks)) for _ in range(nchannels)]
    intra = [list(map(int, row)) for row in intra]
    if len(intra) != nchannels:
        raise ValueError("need one intra-node order per channel")
    for row in intra:
        if len(row) != nranks:
            raise ValueError("an intra-node order lists every rank once")
        for m in range(nnodes):
            if sorted(row[m * L:(m + 1) * L]) != list(range(m * L, (m + 1) * L)):
                raise ValueError(f"order of node {m} is not a permutation of its ranks")
    return intra


def build_topology(nranks: int, nnodes: int, nchannels: int, pattern: str = "tree",
                   intra=None) -> Topology:
    """Per-channel tree records for N ranks on M nodes (L = N/M per node).

    Ranks are node-major: rank = node*L + local.  ``intra[c]`` lists, node
    after node, the ranks of each node in channel c's chain order (default:
    identity).  Inside each node the ranks form a chain in that order: parent
    = previous, first child = next (section "节点内先形成链").  The node-level
    edges of the channel's tree then go to the heads that ``pattern`` names:
    each node's parent head links up to the parent node's child0 or child1
    head (by the node's child type); each node's child0 and child1 heads take
    the parent heads of the child0 and child1 nodes as children, child0 first,
    each in the first empty slot (section "节点间连接").
    """
    if nranks < 1 or nnodes < 1 or nranks % nnodes != 0:
        raise ValueError("need nranks >= 1, nnodes >= 1 and nnodes dividing nranks")
    if nchannels < 1:
        raise ValueError("need at least one channel")
    L = nranks // nnodes
    pos_parent, pos_child0, pos_child1 = head_positions(pattern)
    if max(pos_parent, pos_child0, pos_child1) >= L:
        raise ValueError(f"pattern {pattern!r} needs at least two ranks per node")
    orders = _check_intra(intra, nranks, nnodes, nchannels)
    depth = L - 1 + log2i(nnodes)
    node_trees = [dtree(nnodes, m) for m in range(nnodes)]
    n_first = (nchannels + 1) // 2
    topo = Topology(nranks, nnodes, nchannels, pattern=pattern)
    for c in range(nchannels):
        t = 0 if c < n_first else 1
        order = orders[c]
        up = [-1] * nranks
        down = [[-1, -1, -1] for _ in range(nranks)]
        chain = [order[m * L:(m + 1) * L] for m in range(nnodes)]
        for m in range(nnodes):
            for i, r in enumerate(chain[m]):
                up[r] = chain[m][i - 1] if i > 0 else -1
                down[r][0] = chain[m][i + 1] if i < L - 1 else -1
        parent_head = [chain[m][pos_parent] for m in range(nnodes)]
        child_head = [(chain[m][pos_child0], chain[m][pos_child1]) for m in range(nnodes)]
        for m in range(nnodes):
            parent, child0, child1, ctype = node_trees[m][t]
            if parent != -1:
                _attach_up(up, parent_head[m], child_head[parent][ctype])
            if child0 != -1:
                _attach_down(down, child_head[m][0], parent_head[child0])
            if child1 != -1:
                _attach_down(down, child_head[m][1], parent_head[child1])
        topo.channels.append(ChannelTree(up, down, t, depth, order=list(order)))
    return topo


def check_tree(ch: ChannelTree) -> None:
    """The structural assertions of section "从 GRAPH 日志复原 active tree" plus
    the arity bounds of section "数据结构不是纯二叉树".  Raises TopologyError."""
    n = len(ch.up)
    for r in range(n):
        u = ch.up[r]
        if u != -1 and r not in ch.down[u]:
            raise TopologyError(f"rank {r}: parent {u} does not list it as a child")
        for c in ch.children(r):
            if ch.up[c] != r:
                raise TopologyError(f"rank {r}: child {c} names parent {ch.up[c]}")
    roots = [r for r in range(n) if ch.up[r] == -1]
    if len(roots) != 1:
        raise TopologyError(f"{len(roots)} roots")
    edges = sum(len(ch.children(r)) for r in range(n))
    if edges != n - 1:
        raise TopologyError(f"{edges} edges for {n} ranks")
    for r in range(n):
        seen, x = set(), r
        while ch.up[x] != -1:
            if x in seen:
                raise TopologyError(f"cycle through rank {x}")
            seen.add(x)
            x = ch.up[x]
        if x != roots[0]:
            raise TopologyError(f"rank {r} does not reach the root")
    for r in range(n):
        limit = 2 if ch.up[r] == -1 else 3
        if len(ch.children(r)) > limit:
            raise TopologyError(f"rank {r} has {len(ch.children(r))} children")


def interior_nodes(n: int, which: int) -> set[int]:
    """Node indices with at least one child in tree ``which`` of dtree(n, .).

    "Interior" counts the root when it has a child: this is the reading under
    which the probe table of section "直接执行源码中的 DTree" lists node 0 as
    the shared interior node for odd n.
    """
    out = set()
    for m in range(n):
        _, c0, c1, _ = dtree(n, m)[which]
        if c0 != -1 or c1 != -1:
            out.add(m)
    return out


def node_tree_depth(n: int, which: int) -> int:
    """Longest root-to-leaf path of node-level tree ``which``."""
    best = 0
    for m in range(n):
        d, x = 0, m
        while True:
            p = dtree(n, x)[which][0]
            if p == -1:
                break
            x = p
            d += 1
            if d > n:
                raise TopologyError("cycle in node-level tree")
        best = max(best, d)
    return best


def node_tree_root(n: int, which: int) -> int:
    roots = [m for m in range(n) if dtree(n, m)[which][0] == -1]
    if len(roots) != 1:
        raise TopologyError(f"{len(roots)} node-level roots")
    return roots[0]
