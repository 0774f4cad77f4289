"""Oracle: how one all-reduce message is split over channels, chunks and
rank-chunks (test infrastructure only).

Sources (page title, then section):

* "NCCL 专家课程 13：Tree、双树、层次化连接与真实交叉区间", section "前置知识"
  (each channel owns a disjoint part of the message, named by a grid offset,
  a channel element count and a chunk element count; channels do not repeat
  the message) and section "runTreeSplit 如何流水" (the tree walks its channel
  range chunk by chunk, each chunk at most ``chunkCount`` elements, the last
  one shorter).
* "NCCL 内部机制：一次 AllReduce 如何变成拓扑图、Channel 与 GPU Kernel", section
  "Chunk、slice、step 是三个尺度" (the message is first split across channels,
  then into chunks that move along the ring or tree).
* "all-reduce 每张卡要发多少数据? ring 和 tree 有什么区别?", section "手撕代码"
  (the ring splits the vector into n nearly equal parts, the first parts one
  element longer, as ``numpy.array_split`` does).

PARITY UNPINNED BY THE PAGES for the exact split rule: the pages name the
fields but do not print the body that fills them.  The reading used here (and
listed in the design doc):

* The message is cut into ``unit``-element units (16 bytes); the units are
  dealt to channels like ``array_split`` (the first ``units % nch`` channels
  get one more).  Offsets are clipped to ``count``, so only the very last
  range can end off a unit boundary and trailing channels may be empty.
* Tree: chunks of ``chunk_count`` elements inside each channel range.
* Ring: inside each channel range, loops of ``nranks * chunk_count``
  elements (the last loop shorter); each loop is cut into ``nranks``
  rank-chunks by ``array_split`` over its units.

What pins it anyway (tests/test_oracle_partition.py): coverage and
disjointness invariants, unit alignment, and with ``unit = 1`` the rank-chunk
sizes reduce to ``numpy.array_split``, the interview page's split.
"""

from __future__ import annotations


def split_units(nunits: int, nparts: int) -> list[int]:
    """Sizes of ``nparts`` parts of ``nunits`` items, the first
    ``nunits % nparts`` parts one item larger."""
    base, extra = divmod(nunits, nparts)
    return [base + (1 if p < extra else 0) for p in range(nparts)]


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def channel_ranges(count: int, unit: int, nchannels: int) -> list[tuple[int, int]]:
    """(grid_offset, channel_count) for each channel."""
    sizes = split_units(ceil_div(count, unit), nchannels)
    out, u0 = [], 0
    for nu in sizes:
        start = min(u0 * unit, count)
        end = min((u0 + nu) * unit, count)
        out.append((start, end - start))
        u0 += nu
    return out


def tree_chunks(grid_offset: int, channel_count: int, chunk_count: int) -> list[tuple[int, int]]:
    """(offset, nelem) of each chunk the tree walks in one channel."""
    out = []
    elem = 0
    while elem < channel_count:
        out.append((grid_offset + elem, min(chunk_count, channel_count - elem)))
        elem += chunk_count
    return out


def ring_loops(grid_offset: int, channel_count: int, nranks: int, chunk_count: int,
               unit: int) -> list[list[tuple[int, int]]]:
    """For each ring loop of one channel: the ``nranks`` rank-chunks as
    (offset, nelem), rank-chunk k being the block whose fold starts at rank k."""
    loop_size = nranks * chunk_count
    loops = []
    start = 0
    while start < channel_count:
        length = min(loop_size, channel_count - start)
        sizes = split_units(ceil_div(length, unit), nranks)
        blocks, u0 = [], 0
        for nu in sizes:
            s = min(u0 * unit, length)
            e = min((u0 + nu) * unit, length)
            blocks.append((grid_offset + start + s, e - s))
            u0 += nu
        loops.append(blocks)
        start += loop_size
    return loops
