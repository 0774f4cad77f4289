"""Oracle: standalone reduce-scatter and all-gather, the two halves of the
ring all-reduce (test infrastructure only).

Sources (page title, then section / figure):

* "all-reduce 每张卡要发多少数据? ring 和 tree 有什么区别?", section "先弄清楚:
  每个概念是什么" (reduce-scatter leaves each rank only the one 1/n segment it
  is responsible for, all-gather puts the segments back together; the two
  in a row are an all-reduce), Figure 1 and section "手撕代码" (the steps of
  each half: ``oracle.ring``).
* "NCCL代码分析", section "通讯时如何选择Channel" (the table of collectives and
  algorithms: reduce-scatter and all-gather run on the ring only).
* "NCCL 专家课程 13", section "前置知识" (each channel owns a disjoint part of
  the data) and section "runTreeSplit 如何流水" (the chunk loop inside a
  channel's part).

Readings (listed in the design doc):

* Layout as in the public collectives: reduce-scatter takes N blocks of
  ``recvcount`` elements from every rank and leaves the reduction of block r
  on rank r; all-gather takes ``sendcount`` elements from every rank and
  leaves rank k's data in block k of every rank's output.
* The ring's reduce-scatter leaves position p with block (p+1) mod N; that
  block is made rank order[p]'s own block, so that every rank ends with its
  own block.  In ring order, block r is therefore folded starting at the
  position after r's and ending at r.  All-gather starts each position with
  its own data in that same slot.
* The channels split one block (``channel_ranges`` over ``recvcount`` or
  ``sendcount``); inside a channel the ring steps run chunk by chunk
  (``chunk_bytes``), each step moving the same piece of every block.
  Chunking never changes an element's order.

Pins (tests/test_oracle_collectives.py): brute force for integer sums, max
and all-gather copies; a hand-derived float order pin; reduce-scatter
followed by all-gather equals the ring all-reduce bit for bit; per-rank send
volumes (n-1) blocks per half.
"""

from __future__ import annotations

import numpy as np

from . import numerics, partition, ring, topology


def _orders(nranks, nnodes, nchannels, intra):
    return [ch.order for ch in topology.build_topology(nranks, nnodes, nchannels, "tree", intra).channels]


def _unit(dtype: str) -> int:
    return max(1, 16 // numerics.ITEMSIZE[dtype])


def reduce_scatter(inputs: list[np.ndarray], nnodes: int, nchannels: int, chunk_bytes: int,
                   dtype: str, op: str, intra=None, stats: dict | None = None) -> list[np.ndarray]:
    """``inputs[r]`` holds N blocks of recvcount elements; returns rank r's
    reduced block r for every r."""
    n = len(inputs)
    total = len(inputs[0])
    if total % n:
        raise ValueError("reduce-scatter input must hold nranks blocks")
    rc = total // n
    want = numerics.STORAGE[dtype]
    if any(x.dtype != want or len(x) != total for x in inputs):
        raise ValueError("every rank needs the same count and storage dtype")
    chunk = chunk_bytes // numerics.ITEMSIZE[dtype]
    orders = _orders(n, nnodes, nchannels, intra)
    out = [np.empty(rc, dtype=want) for _ in range(n)]
    sent = [0] * n

    def comb(a, b):
        return numerics.combine(dtype, op, a, b)

    for c, (off, ln) in enumerate(partition.channel_ranges(rc, _unit(dtype), nchannels)):
        order = orders[c]
        data_block = [order[(k - 1) % n] for k in range(n)]   # step-schedule block k -> data block
        for o, piece in partition.tree_chunks(off, ln, chunk):
            bufs = [[inputs[order[p]][data_block[k] * rc + o: data_block[k] * rc + o + piece].copy()
                     for k in range(n)] for p in range(n)]
            pos_sent = [0] * n
            ring.ring_reduce_scatter_steps(bufs, comb, lambda a: a.copy(), sent=pos_sent, size=len)
            for p in range(n):
                sent[order[p]] += pos_sent[p]
                out[order[p]][o:o + piece] = bufs[p][(p + 1) % n]
    if stats is not None:
        stats["sent_elems"] = sent
    return out


def all_gather(inputs: list[np.ndarray], nnodes: int, nchannels: int, chunk_bytes: int, dtype: str,
               intra=None, stats: dict | None = None) -> list[np.ndarray]:
    """``inputs[r]`` holds sendcount elements; returns for every rank the N
    blocks, block k holding rank k's data."""
    n = len(inputs)
    sc = len(inputs[0])
    want = numerics.STORAGE[dtype]
    if any(x.dtype != want or len(x) != sc for x in inputs):
        raise ValueError("every rank needs the same count and storage dtype")
    chunk = chunk_bytes // numerics.ITEMSIZE[dtype]
    orders = _orders(n, nnodes, nchannels, intra)
    out = [np.empty(n * sc, dtype=want) for _ in range(n)]
    sent = [0] * n
    for c, (off, ln) in enumerate(partition.channel_ranges(sc, _unit(dtype), nchannels)):
        order = orders[c]
        data_block = [order[(k - 1) % n] for k in range(n)]
        for o, piece in partition.tree_chunks(off, ln, chunk):
            bufs = [[None] * n for _ in range(n)]
            for p in range(n):
                bufs[p][(p + 1) % n] = inputs[order[p]][o:o + piece].copy()
            pos_sent = [0] * n
            ring.ring_all_gather_steps(bufs, lambda a: a.copy(), sent=pos_sent, size=len)
            for p in range(n):
                sent[order[p]] += pos_sent[p]
                for k in range(n):
                    d = data_block[k]
                    out[order[p]][d * sc + o: d * sc + o + piece] = bufs[p][k]
    if stats is not None:
        stats["sent_elems"] = sent
    return out
