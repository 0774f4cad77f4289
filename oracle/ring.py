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
  - section "手撕代码" (at reduce-scatter step s rank r sends block (r-s) mod n
    to rank r+1; at all-gather step s it sends block (r+1-s) mod n; every rank
    copies what it sends before any receiver applies its update, so all sends
    of a step read the values from before that step).
* "NCCL 内部机制：一次 AllReduce 如何变成拓扑图、Channel 与 GPU Kernel", section
  "Ring：带宽友好，但启动步骤会随规模增长" (first step sends, middle steps
  receive-reduce-send, the last reduce-scatter step also writes the result,
  then the finished blocks are forwarded around the ring).

The simulator moves whole blocks between per-rank block lists.  It is
generic in what a block is: numpy arrays with the rounding ``combine`` of
``numerics`` for numbers, or frozensets with set union for the symbolic
contributor tables of Figure 1.

Consequence used by the tests: block k's value is the left fold that starts
at rank k and walks the ring, x_k, x_{k+1}, ..., x_{k-1}, each hop rounded.
(The receiver computes own (op) incoming; a single rounded add or max is
commutative, so this is the same bits as incoming (op) own.)
"""

from __future__ import annotations

from typing import Any, Callable


def ring_reduce_scatter_steps(bufs: list[list[Any]], combine: Callable[[Any, Any], Any],
                              copy: Callable[[Any], Any], trace: list | None = None,
                              sent: list[int] | None = None, size: Callable[[Any], int] | None = None) -> None:
    """The n-1 reduce-scatter steps, in place on ``bufs[r][b]`` (position r,
    block b): at step s every position r sends block (r-s) mod n to r+1,
    which adds it to its own copy of that block; all sends of a step read the
    values from before the step.  Afterwards position r holds the full
    reduction of block (r+1) mod n.  ``trace``/``sent``/``size`` as in
    :func:`ring_allreduce_blocks`."""
    n = len(bufs)
    for s in range(n - 1):
        outgoing = [copy(bufs[r][(r - s) % n]) for r in range(n)]
        for r in range(n):
            dst, b = (r + 1) % n, (r - s) % n
            bufs[dst][b] = combine(bufs[dst][b], outgoing[r])
            if sent is not None:
                sent[r] += size(outgoing[r])
        if trace is not None:
            trace.append((("RS", s + 1), [[copy(b) for b in row] for row in bufs]))


def ring_all_gather_steps(bufs: list[list[Any]], copy: Callable[[Any], Any], trace: list | None = None,
                          sent: list[int] | None = None, size: Callable[[Any], int] | None = None) -> None:
    """The n-1 all-gather steps, in place: position r starts with (at least)
    block (r+1) mod n; at step s it sends block (r+1-s) mod n to r+1, which
    overwrites its copy.  Afterwards every position holds every block."""
    n = len(bufs)
    for s in range(n - 1):
        outgoing = [copy(bufs[r][(r + 1 - s) % n]) for r in range(n)]
        for r in range(n):
            dst, b = (r + 1) % n, (r + 1 - s) % n
            bufs[dst][b] = outgoing[r]
            if sent is not None:
                sent[r] += size(outgoing[r])
        if trace is not None:
            trace.append((("AG", s + 1), [[copy(b) if b is not None else None for b in row] for row in bufs]))


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
