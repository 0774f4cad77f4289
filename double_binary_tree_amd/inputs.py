"""Seeded synthetic inputs and the named workloads.

This module holds no reduction arithmetic: it only draws per-rank input
arrays (numpy ``PCG64``; per-rank streams from ``SeedSequence.spawn``) and
describes the workload shapes.  Both the oracle tests and the GPU path take
their inputs from here.

The workloads mirror the message-size sweeps of the pages' measurements
(nccl-tests ``all_reduce_perf``: power-of-two per-rank sizes, sum, out-of-place
and in-place), with the rank counts, node counts, channel counts, element
types and value distributions fixed for this build.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

SEED_BASE = 20261202

_STORAGE = {"i32": np.int32, "i64": np.int64, "f32": np.float32,
            "f16": np.float16, "bf16": np.uint16}
_ITEMSIZE = {"i32": 4, "i64": 8, "f32": 4, "f16": 2, "bf16": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    seed_index: int          # seed = SEED_BASE + seed_index
    nranks: int
    nnodes: int
    algos: tuple             # ("ring",), ("tree",) or both
    nchannels: int
    chunk_bytes: int
    dtype: str
    op: str
    count: int               # elements per rank
    dist: tuple              # ("int", lo, hi) | ("normal", sigma) | ("uniform", lo, hi)

    @property
    def itemsize(self) -> int:
        return _ITEMSIZE[self.dtype]

    @property
    def bytes_per_rank(self) -> int:
        return self.count * self.itemsize

    def with_count(self, count: int) -> "Workload":
        return replace(self, count=count)


KiB = 1024
MiB = 1024 * 1024

WORKLOADS = {
    # 4 ranks, one node, ring, one channel: the 4-rank step table shape.
    "ring4_i32": Workload("ring4_i32", 1, 4, 1, ("ring",), 1, 512 * KiB, "i32", "sum",
                          1024, ("int", -1000, 1000)),
    # 8 ranks on one node (the tree is the intra-node chain), 12 channels.
    "chain8_f32": Workload("chain8_f32", 2, 8, 1, ("ring", "tree"), 12, 512 * KiB, "f32", "sum",
                           16 * MiB, ("normal", 1.0)),
    # Double binary tree over 16 single-rank nodes (even: mirror).
    "dtree16_bf16": Workload("dtree16_bf16", 3, 16, 16, ("tree",), 8, 512 * KiB, "bf16", "sum",
                             16 * MiB, ("normal", 1.0)),
    # Double binary tree over 15 single-rank nodes (odd: shift).
    "dtree15_bf16": Workload("dtree15_bf16", 3, 15, 15, ("tree",), 8, 512 * KiB, "bf16", "sum",
                             16 * MiB, ("normal", 1.0)),
    # Ring vs tree sweep shape (count and channels vary per point).
    "sweep8_f32": Workload("sweep8_f32", 4, 8, 1, ("ring", "tree"), 12, 512 * KiB, "f32", "sum",
                           1 << 20, ("uniform", -1.0, 1.0)),
    # Hierarchical: 4 nodes x 8 local ranks, chain inside, double tree across.
    "hier4x8_f16": Workload("hier4x8_f16", 5, 32, 4, ("tree",), 16, 512 * KiB, "f16", "sum",
                            8 * MiB, ("normal", 0.1)),
    "hier4x8_i64": Workload("hier4x8_i64", 5, 32, 4, ("tree",), 16, 512 * KiB, "i64", "sum",
                            8 * MiB, ("int", -(1 << 40), 1 << 40)),
    "hier4x8_f32max": Workload("hier4x8_f32max", 5, 32, 4, ("tree",), 16, 512 * KiB, "f32", "max",
                               8 * MiB, ("normal", 1.0)),
}

SWEEP_CHANNELS = (1, 4, 12, 32)
SWEEP_COUNTS = tuple(1 << p for p in range(1, 27))   # 8 B .. 256 MiB of f32


def _round_f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Input preparation only: round drawn float32 values to bf16 with torch's
    CPU conversion (round to nearest even) and return the bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def draw(rng: np.random.Generator, dtype: str, dist: tuple, count: int) -> np.ndarray:
    kind = dist[0]
    if kind == "int":
        lo, hi = dist[1], dist[2]
        return rng.integers(lo, hi, size=count, endpoint=True, dtype=np.int64).astype(_STORAGE[dtype])
    if kind == "normal":
        x = rng.standard_normal(count, dtype=np.float32) * np.float32(dist[1])
    elif kind == "uniform":
        x = rng.uniform(dist[1], dist[2], size=count).astype(np.float32)
    else:
        raise ValueError(f"unknown distribution {dist}")
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return _round_f32_to_bf16_bits(x)
    raise ValueError(f"float distribution for integer dtype {dtype}")


def rank_inputs(w: Workload, count: int | None = None, salt: int = 0) -> list[np.ndarray]:
    """One input array per rank for workload ``w`` (optionally resized).

    ``salt`` picks an independent stream family (used for extra test cases)."""
    n = w.count if count is None else count
    seed = SEED_BASE + w.seed_index + 1000 * salt
    children = np.random.SeedSequence(seed).spawn(w.nranks)
    return [draw(np.random.Generator(np.random.PCG64(ch)), w.dtype, w.dist, n) for ch in children]


# Float layouts: (storage bits, exponent bits, significand bits).
_FLOAT_BITS = {"f32": (32, 8, 23), "f16": (16, 5, 10), "bf16": (16, 8, 7)}

SPECIAL_TINY, SPECIAL_MIXED, SPECIAL_HUGE, SPECIAL_INF = 0, 1, 2, 3


def special_inputs(nranks: int, dtype: str, count: int, seed: int):
    """Inputs made of IEEE special values, built bit by bit (float types only).

    Every position gets a class and a sign, shared by all ranks:
      SPECIAL_TINY   every rank holds a subnormal or a zero of random sign,
                     with a significand below 2**(m-6) (m significand bits),
                     so any sum of up to 64 of them stays subnormal and exact;
      SPECIAL_MIXED  each rank holds a zero, a subnormal (any significand) or
                     a normal number of magnitude about 1, of random sign;
      SPECIAL_HUGE   two distinct ranks hold numbers of the largest finite
                     binade with the position's sign, the others mixed
                     values (one rank: mixed);
      SPECIAL_INF    one rank holds infinity with the position's sign, every
                     other rank infinity of that sign with probability 1/5,
                     else a mixed value.
    No NaN, and no position holds infinities or largest-binade numbers of
    both signs, so no sum can produce a NaN.

    Returns (inputs, cls, sign): one array per rank in the storage type
    (bf16 as uint16 bits), and the per-position class and sign (1 = negative).
    """
    width, ebits, mbits = _FLOAT_BITS[dtype]
    utype = np.uint32 if width == 32 else np.uint16
    emax = (1 << ebits) - 1                 # all-ones exponent: infinity
    bias = (1 << (ebits - 1)) - 1
    children = np.random.SeedSequence(SEED_BASE + 7000 + seed).spawn(nranks + 1)
    shared = np.random.Generator(np.random.PCG64(children[-1]))
    cls = shared.integers(0, 4, size=count)
    if nranks == 1:
        cls = np.where(cls == SPECIAL_HUGE, SPECIAL_MIXED, cls)
    sign = shared.integers(0, 2, size=count)
    first = shared.integers(0, nranks, size=count)
    second = (first + 1 + shared.integers(0, max(nranks - 1, 1), size=count)) % nranks

    def pack(sg, ex, mant):
        return ((sg.astype(np.uint64) << (width - 1)) | (ex.astype(np.uint64) << mbits) |
                mant.astype(np.uint64)).astype(utype)

    out = []
    for r in range(nranks):
        rng = np.random.Generator(np.random.PCG64(children[r]))
        rsign = rng.integers(0, 2, size=count)
        mant = rng.integers(0, 1 << mbits, size=count)
        kind = rng.integers(0, 3, size=count)          # mixed: 0 zero, 1 subnormal, 2 normal
        ex = np.where(kind == 2, bias + rng.integers(-4, 5, size=count), 0)
        mant = np.where(kind == 0, 0, mant)
        bits = pack(rsign, ex, mant)
        tiny = pack(rsign, np.zeros(count, dtype=np.int64), rng.integers(0, 1 << (mbits - 6) if mbits > 6 else 2,
                                                                         size=count))
        huge = pack(sign, np.full(count, emax - 1), rng.integers(0, 1 << mbits, size=count))
        inf = pack(sign, np.full(count, emax), np.zeros(count, dtype=np.int64))
        bits = np.where(cls == SPECIAL_TINY, tiny, bits)
        is_huge = (cls == SPECIAL_HUGE) & ((first == r) | (second == r))
        bits = np.where(is_huge, huge, bits)
        is_inf = (cls == SPECIAL_INF) & ((first == r) | (rng.random(count) < 0.2))
        bits = np.where(is_inf, inf, bits)
        if dtype == "f32":
            out.append(bits.view(np.float32))
        elif dtype == "f16":
            out.append(bits.view(np.float16))
        else:
            out.append(bits)
    return out, cls, sign


def intra_orders(nranks: int, nnodes: int, nchannels: int, seed: int, distinct: int = 3) -> list[list[int]]:
    """Seeded per-channel rank orders for graph test cases: each channel takes
    one of ``distinct`` random orders, each a permutation of every node's
    ranks, node after node (rank = node * L + local)."""
    rng = np.random.default_rng(SEED_BASE + seed)
    L = nranks // nnodes
    pool = [[int(r) for m in range(nnodes) for r in rng.permutation(range(m * L, (m + 1) * L))]
            for _ in range(distinct)]
    return [pool[int(rng.integers(0, distinct))] for _ in range(nchannels)]
