"""Oracle: one whole all-reduce over N virtual ranks (test infrastructure only).

Puts the pieces together the way the pages describe the data path:

* "NCCL 专家课程 13", section "为什么不是发送两份完整消息": each channel
  handles its own part of the message on its own tree; channel parts are
  disjoint.
* Ring: per channel, per loop, the rank-chunks go through the ring steps of
  ``oracle.ring``.
* Tree: per channel, per chunk, the ranks run the reduce-up/broadcast-down
  of ``oracle.tree`` on that channel's tree record from ``oracle.topology``.

Also here: the float64 reference sum, the normwise tolerance the float
results are held to, and the rigorous elementwise rounding-error bound that
any rounded fold of N values obeys.

Everything is plain numpy on host arrays, slow on purpose.
"""

from __future__ import annotations

import numpy as np

from . import numerics, partition, ring, topology, tree

ALGOS = ("ring", "tree")
UNIT_BYTES = 16


def _check_inputs(inputs, dtype):
    n = len(inputs)
    if n < 1:
        raise ValueError("need at least one rank")
    count = len(inputs[0])
    want = numerics.STORAGE[dtype]
    for x in inputs:
        if x.dtype != want or len(x) != count:
            raise ValueError("every rank needs the same count and storage dtype")
    return n, count


def _element_unit(dtype: str, unit_bytes: int) -> int:
    esz = numerics.ITEMSIZE[dtype]
    return max(1, unit_bytes // esz)


def allreduce(inputs: list[np.ndarray], nnodes: int, algo: str, nchannels: int,
              chunk_bytes: int, dtype: str, op: str, unit_bytes: int = UNIT_BYTES,
              stats: dict | None = None, pattern: str = "tree", intra=None) -> list[np.ndarray]:
    """All-reduce ``inputs`` (one array per rank); returns one array per rank.

    ``pattern`` and ``intra`` (per-channel rank orders) are passed to
    :func:`oracle.topology.build_topology`.  The ring of channel c visits the
    ranks in ``intra[c]`` order: ring position p is rank ``intra[c][p]``, and
    the ring steps of ``oracle.ring`` run over positions.
    ``stats``, if given, receives ``sent_elems`` (per-rank elements sent).
    """
    n, count = _check_inputs(inputs, dtype)
    outputs = [np.array(x, copy=True) for x in inputs]
    sent = [0] * n
    topo = topology.build_topology(n, nnodes, nchannels, pattern, intra)
    for c in range(nchannels):
        allreduce_channel(inputs, outputs, c, topo, algo, chunk_bytes, dtype, op, unit_bytes, sent)
    if stats is not None:
        stats["sent_elems"] = sent
    return outputs


def allreduce_channel(inputs: list[np.ndarray], outputs: list[np.ndarray], c: int, topo, algo: str,
                      chunk_bytes: int, dtype: str, op: str, unit_bytes: int = UNIT_BYTES,
                      sent: list[int] | None = None) -> None:
    """Channel c's part of the all-reduce: writes its element range of every
    rank's ``outputs``; the channels' ranges are disjoint, so they can be
    computed in any order (or at the same time).  ``topo`` is the
    communicator's :func:`oracle.topology.build_topology`."""
    n, count = _check_inputs(inputs, dtype)
    esz = numerics.ITEMSIZE[dtype]
    unit = _element_unit(dtype, unit_bytes)
    if chunk_bytes % esz:
        raise ValueError("chunk_bytes must hold whole elements")
    chunk_count = chunk_bytes // esz

    def comb(a, b):
        return numerics.combine(dtype, op, a, b)

    def cp(a):
        return np.array(a, copy=True)

    grid_offset, ch_count = partition.channel_ranges(count, unit, topo.nchannels)[c]
    if algo == "ring":
        order = topo.channels[c].order
        for blocks in partition.ring_loops(grid_offset, ch_count, n, chunk_count, unit):
            bufs = [[inputs[order[p]][o:o + ln].copy() for (o, ln) in blocks] for p in range(n)]
            pos_sent = [0] * n
            ring.ring_allreduce_blocks(bufs, comb, cp, sent=pos_sent, size=len)
            for p in range(n):
                if sent is not None:
                    sent[order[p]] += pos_sent[p]
                for (o, ln), blk in zip(blocks, bufs[p]):
                    outputs[order[p]][o:o + ln] = blk
    elif algo == "tree":
        ch = topo.channels[c]
        for o, ln in partition.tree_chunks(grid_offset, ch_count, chunk_count):
            res = tree.tree_allreduce_chunk([inputs[r][o:o + ln] for r in range(n)],
                                            ch.up, ch.down, comb, cp, sent=sent, size=len)
            for r in range(n):
                outputs[r][o:o + ln] = res[r]
    else:
        raise ValueError(f"unknown algo {algo}")


def allreduce_at(inputs: list[np.ndarray], index: np.ndarray, nnodes: int, algo: str,
                 nchannels: int, chunk_bytes: int, dtype: str, op: str,
                 unit_bytes: int = UNIT_BYTES, pattern: str = "tree", intra=None) -> np.ndarray:
    """The all-reduce result at element positions ``index`` only.

    Each position is placed in its channel and loop/chunk by the same
    partition as :func:`allreduce`, and the same ring or tree simulator runs
    on just the sampled positions of each block (every step is elementwise,
    so restricting a block to some of its positions gives those positions'
    exact values).  Lets the tests check full-size runs position by position.
    """
    n, count = _check_inputs(inputs, dtype)
    esz = numerics.ITEMSIZE[dtype]
    unit = _element_unit(dtype, unit_bytes)
    chunk_count = chunk_bytes // esz
    index = np.asarray(index, dtype=np.int64)
    if index.size and (index.min() < 0 or index.max() >= count):
        raise ValueError("index out of range")
    out = np.empty(index.shape, dtype=numerics.STORAGE[dtype])
    done = np.zeros(index.shape, dtype=bool)

    def comb(a, b):
        return numerics.combine(dtype, op, a, b)

    def cp(a):
        return np.array(a, copy=True)

    ranges = partition.channel_ranges(count, unit, nchannels)
    topo = topology.build_topology(n, nnodes, nchannels, pattern, intra)
    for c, (grid_offset, ch_count) in enumerate(ranges):
        in_ch = (index >= grid_offset) & (index < grid_offset + ch_count)
        if not in_ch.any():
            continue
        if algo == "ring":
            for blocks in partition.ring_loops(grid_offset, ch_count, n, chunk_count, unit):
                sel = [np.nonzero((index >= o) & (index < o + ln))[0] for (o, ln) in blocks]
                if not any(s.size for s in sel):
                    continue
                order = topo.channels[c].order
                bufs = [[inputs[order[p]][index[s]] for s in sel] for p in range(n)]
                ring.ring_allreduce_blocks(bufs, comb, cp)
                for s, blk in zip(sel, bufs[0]):
                    out[s] = blk
                    done[s] = True
        elif algo == "tree":
            ch = topo.channels[c]
            where = np.nonzero(in_ch)[0]
            res = tree.tree_allreduce_chunk([inputs[r][index[where]] for r in range(n)],
                                            ch.up, ch.down, comb, cp)
            out[where] = res[0]
            done[where] = True
        else:
            raise ValueError(f"unknown algo {algo}")
    if not done.all():
        raise AssertionError("partition left positions uncovered")
    return out


def reference_sum(inputs: list[np.ndarray], dtype: str, index=None):
    """Exact sum over ranks for integers (Python ints via object arrays);
    float64 sum of the exact values for floats."""
    sel = (lambda x: x) if index is None else (lambda x: x[index])
    if numerics.is_float(dtype):
        acc = np.zeros(len(sel(inputs[0])), dtype=np.float64)
        for x in inputs:
            acc += numerics.to_f64(sel(x), dtype)
        return acc
    acc = np.zeros(len(sel(inputs[0])), dtype=object)
    for x in inputs:
        acc = acc + sel(x).astype(object)
    return acc


def abs_sum(inputs: list[np.ndarray], dtype: str, index=None) -> np.ndarray:
    sel = (lambda x: x) if index is None else (lambda x: x[index])
    acc = np.zeros(len(sel(inputs[0])), dtype=np.float64)
    for x in inputs:
        acc += np.abs(numerics.to_f64(sel(x), dtype))
    return acc


UNIT_ROUNDOFF = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
# Half the spacing of the smallest subnormals: the absolute error one rounding
# can add when a partial falls in the subnormal range.
UNDERFLOW_HALF_SPACING = {"f32": 2.0 ** -150, "f16": 2.0 ** -25, "bf16": 2.0 ** -134}


def normwise_error(result: np.ndarray, inputs: list[np.ndarray], dtype: str, index=None) -> float:
    """Normwise relative error of the result vector: ||y - s64||_2 / ||s64||_2."""
    s64 = reference_sum(inputs, dtype, index)
    y = numerics.to_f64(result, dtype)
    den = float(np.sqrt(np.sum(s64 * s64)))
    num = float(np.sqrt(np.sum((y - s64) ** 2)))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


def within_tolerance(result: np.ndarray, inputs: list[np.ndarray], dtype: str,
                     rtol: float, index=None) -> tuple[bool, float]:
    """Float sums: the normwise relative error of the vector is at most rtol.

    (Reading of the "1e-5 relative (fp32) / 1e-2 (bf16, fp16) against an fp64
    sum" target: per element, a relative error is meaningless where the
    signed sum cancels, and an error scaled by sum_r |x_r| can legitimately
    exceed 1e-2 for bf16 after several rounded hops; the vector norm is the
    usual meaning of a relative error of a result vector.)
    Returns (ok, error)."""
    err = normwise_error(result, inputs, dtype, index)
    return err <= rtol, err


def within_rounding_bound(result: np.ndarray, inputs: list[np.ndarray], dtype: str,
                          index=None) -> tuple[bool, float]:
    """Elementwise rigorous bound for any fold of N values with N-1 rounded
    operations: |y - s64| <= gamma_{N-1} * sum_r |x_r| + (N-1) * eta, where
    gamma_h = h*u / (1 - h*u), u the unit roundoff of the buffer type and eta
    half the smallest subnormal spacing (standard floating-point summation
    error analysis).  Returns (ok, worst |y - s64| / bound)."""
    n = len(inputs)
    h = max(n - 1, 0)
    u = UNIT_ROUNDOFF[dtype]
    gamma = h * u / (1 - h * u)
    s64 = reference_sum(inputs, dtype, index)
    scale = abs_sum(inputs, dtype, index)
    y = numerics.to_f64(result, dtype)
    bound = gamma * scale + h * UNDERFLOW_HALF_SPACING[dtype]
    err = np.abs(y - s64)
    ok = bool(np.all(err <= bound))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    return ok, float(ratio.max()) if ratio.size else 0.0
