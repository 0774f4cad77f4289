"""Oracle: ring all-reduce as reduce-scatter followed by all-gather
(test infrastructure only).

Sources (page title, then section / figure):

* "all-reduce 每张卡要发多少数据? ring 和 tree 有什么区别?":
  - section "先弄清楚:每个概念是什么" (all-reduce = reduce-scatter, after which
    each rank holds one fully reduced 1/n part, then all-gather);
  - Figure 1 (4 ranks, every step each rank passes one block to its right
    neighbour; in reduce-scatter the receiver adds it to its own block, in
    all-gather the receiver overwrites its block with the finished sum);
  - section "推导 / 关键公式" (each rank sends 2(n-1) blocks of S/n);
  - section "手撕代码" (the same schedule simulated step by step: all sends of
    a step read the values from before that step).
* "NCCL 内部机制：一次 AllReduce 如何变成拓扑图、Channel 与 GPU Kernel", section
  "Ring：带宽友好，但启动步骤会随规模增长" (first step sends, middle steps
  receive-reduce-send, the last reduce-scatter step also writes the result,
  then the finished blocks are forwarded around the ring).

The simulator follows each block along its route round the ring (the
positions it visits, one hop per step) and moves whole blocks between
per-position block lists.  It is generic in what a block is: numpy arrays
with the rounding ``combine`` of ``numerics`` for numbers, or frozensets
with set union for the symbolic contributor tables of Figure 1.

Consequence used by the tests: block k's value is the left fold that starts
at rank k and walks the ring, x_k, x_{k+1}, ..., x_{k-1}, each hop rounded.
(The receiver computes own (op) incoming; a single rounded add or max is
commutative, so this is the same bits as incoming (op) own.)
"""

from __future__ import annotations

from typing import Any, Callable


def ring_route(n: int, k: int) -> list[int]:
    """The positions block k visits in the reduce-scatter: it starts at
    position k (Figure 1: every rank first sends its own block) and moves
    one position along the ring, p -> p+1, at every step."""
    return [(k + j) % n for j in range(n)]


def ring_reduce_scatter_steps(bufs: list[list[Any]], combine: Callable[[Any, Any], Any],
                              copy: Callable[[Any], Any], trace: list | None = None,
                              sent: list[int] | None = None, size: Callable[[Any], int] | None = None) -> None:
    """The n-1 reduce-scatter steps, in place on ``bufs[p][b]`` (position p,
    block b).  At step j every block b takes one hop of its route: the
    position that holds its partial so far, route[j-1], passes it on to
    route[j], which folds it into its own copy (own (op) incoming, rounded).
    One step's hops write cells (route[j], b) and read cells (route[j-1], b),
    never a cell another hop of the step writes, so every hop sees the
    values from before the step.  Afterwards position p holds the full
    reduction of block p+1 (mod n).  ``trace``/``sent``/``size`` as in
    :func:`ring_allreduce_blocks`."""
    n = len(bufs)
    routes = [ring_route(n, b) for b in range(n)]
    for j in range(1, n):
        for b in range(n):
            src, dst = routes[b][j - 1], routes[b][j]
            incoming = copy(bufs[src][b])
            bufs[dst][b] = combine(bufs[dst][b], incoming)
            if sent is not None:
                sent[src] += size(incoming)
        if trace is not None:
            trace.append((("RS", j), [[copy(x) for x in row] for row in bufs]))


def ring_all_gather_steps(bufs: list[list[Any]], copy: Callable[[Any], Any], trace: list | None = None,
                          sent: list[int] | None = None, size: Callable[[Any], int] | None = None) -> None:
    """The n-1 all-gather steps, in place: the finished block b sits at the
    end of its reduce-scatter route, position b-1 (mod n); at step j it
    moves on from position b+j-2 to b+j-1, which overwrites its copy.
    Afterwards every position holds every block."""
    n = len(bufs)
    for j in range(1, n):
        for b in range(n):
            src, dst = (b + j - 2) % n, (b + j - 1) % n
            bufs[dst][b] = copy(bufs[src][b])
            if sent is not None:
                sent[src] += size(bufs[dst][b])
        if trace is not None:
            trace.append((("AG", j), [[copy(x) if x is not None else None for x in row] for row in bufs]))


def ring_allreduce_blocks(bufs: list[list[Any]], combine: Callable[[Any, Any], Any],
                          copy: Callable[[Any], Any],
                          trace: list | None = None,
                          sent: list[int] | None = None,
                          size: Callable[[Any], int] | None = None) -> None:
    """Run the 2(n-1) ring steps in place on ``bufs[r][b]`` (rank r, block b).

    ``trace``, if given, receives a snapshot (list of per-rank block lists,
    copied) after every step, labelled ("RS", s+1) or ("AG", s+1).
    ``sent``, if given, accumulates per rank the ``size`` of every block
    the rank sends.
    """
    n = len(bufs)
    for r in range(n):
        if len(bufs[r]) != n:
            raise ValueError("every rank needs one block per rank")
    ring_reduce_scatter_steps(bufs, combine, copy, trace, sent, size)
    ring_all_gather_steps(bufs, copy, trace, sent, size)
