"""Oracle: tree all-reduce, reduce-up then broadcast-down (test
infrastructure only).

Sources: "NCCL 专家课程 13：Tree、双树、层次化连接与真实交叉区间",
* section "先固定方向": reduce receives from the children, folds in the local
  input and sends to the parent; broadcast receives from the parent, keeps a
  copy and sends to the children;
* section "runTreeSplit 如何流水": a leaf (no first child) only sends its input
  up; an internal rank receives its children, folds in its input and sends
  up; the root receives its children, folds in its input, writes the result
  and sends it down; internal ranks receive the result, write it and pass it
  on; leaves receive it;
* section "每种 rank 的操作": the worked chain 0->1->2->3 (rank 2 adds rank 3's
  input to its own, rank 1 adds that partial to its own, the root adds the
  rest to its own).

Reading where the pages are silent: at a rank with two or more
children the accumulator starts as the rank's own input and the children's
partials are folded in child-slot order, one rounded operation each:
v(r) = (((x_r (op) v(down0)) (op) v(down1)) (op) v(down2)).  With a single
child this is the pages' chain order.  PARITY UNPINNED BY THE PAGES for the
order among two or more children.

Chunking does not change any fold, so the simulator works on whatever
element range it is given.
"""

from __future__ import annotations

from typing import Any, Callable


def tree_allreduce_chunk(inputs: list[Any], up: list[int], down: list[list[int]],
                         combine: Callable[[Any, Any], Any], copy: Callable[[Any], Any],
                         sent: list[int] | None = None,
                         size: Callable[[Any], int] | None = None) -> list[Any]:
    """Reduce-up then broadcast-down of one chunk; returns per-rank outputs."""
    n = len(inputs)
    depth = [0] * n
    for r in range(n):
        x = r
        while up[x] != -1:
            x = up[x]
            depth[r] += 1
    root = [r for r in range(n) if up[r] == -1]
    if len(root) != 1:
        raise ValueError("tree must have exactly one root")
    root = root[0]

    # Reduce-up: a rank folds once every child has sent, so visit deepest first.
    partial: dict[int, Any] = {}
    for r in sorted(range(n), key=lambda q: -depth[q]):
        acc = copy(inputs[r])
        for c in down[r]:
            if c != -1:
                acc = combine(acc, partial[c])
        partial[r] = acc
        if up[r] != -1 and sent is not None:
            sent[r] += size(acc)

    # Broadcast-down: the root's fold is the result; each rank writes what it
    # received and forwards it to its children, shallowest first.
    outputs: list[Any] = [None] * n
    outputs[root] = partial[root]
    for r in sorted(range(n), key=lambda q: depth[q]):
        for c in down[r]:
            if c != -1:
                outputs[c] = copy(outputs[r])
                if sent is not None:
                    sent[r] += size(outputs[r])
    return outputs
