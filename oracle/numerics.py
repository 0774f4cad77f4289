"""Oracle: element types and the reduction operator with per-hop rounding
(test infrastructure only).

Sources: "NCCL 内部机制：一次 AllReduce 如何变成拓扑图、Channel 与 GPU Kernel",
section on the public call ("ncclAllReduce" arguments: element count, data
type, reduction operator such as sum or max); "NCCL 专家课程 13", section "每种
rank 的操作" (every hop receives a partial, reduces it with the local input and
passes the result on, so rounding happens at every hop).

Readings (the pages are silent on rounding; listed in the design doc):

* Every binary reduction is rounded to the buffer type before it is passed
  on.  ``f32``: one IEEE single add (round to nearest even, subnormals kept).
  ``f16`` and ``bf16``: widen both operands to f32, add there, round the f32
  sum to the 16-bit type to nearest even.  Because f32 carries at least
  2p+2 significand bits for p = 8 (bf16) and p = 11 (f16), this equals the
  correctly rounded 16-bit sum.
* Integer sums wrap (two's complement).
* Float max picks the numerically larger operand, with -0 below +0; the
  inputs never hold NaN.  This max is commutative and associative, so its
  result is the plain maximum whatever the order.

``bf16`` values are carried as their uint16 bit patterns (numpy has no bf16).

Pins (tests/test_oracle_numerics.py): bf16 rounding against the nearest
point of the complete sorted bf16 grid, f16 rounding against numpy's own
conversion, the 16-bit sum against the exactly rounded rational sum, and
max against numpy's maximum.
"""

from __future__ import annotations

import numpy as np

DTYPES = ("i32", "i64", "f32", "f16", "bf16")
OPS = ("sum", "max")

STORAGE = {
    "i32": np.dtype(np.int32),
    "i64": np.dtype(np.int64),
    "f32": np.dtype(np.float32),
    "f16": np.dtype(np.float16),
    "bf16": np.dtype(np.uint16),
}

ITEMSIZE = {k: v.itemsize for k, v in STORAGE.items()}


def is_float(dtype: str) -> bool:
    return dtype in ("f32", "f16", "bf16")


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact: bf16 is the top half of f32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 bit patterns, nearest with ties to even.

    The kept part is the upper 16 bits; the dropped part is the lower 16.
    Round up when the dropped part exceeds half an ulp, or equals it and the
    kept part is odd.  A carry out of the significand moves the exponent, and
    past the largest finite value gives infinity, as IEEE rounding requires.
    NaN stays NaN (quiet bit set).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    kept = (u >> np.uint32(16)).astype(np.uint32)
    dropped = u & np.uint32(0xFFFF)
    half = np.uint32(0x8000)
    up = (dropped > half) | ((dropped == half) & ((kept & np.uint32(1)) == 1))
    rounded = kept + up.astype(np.uint32)
    is_nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    rounded = np.where(is_nan, kept | np.uint32(0x0040), rounded)
    return rounded.astype(np.uint16)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements (float types only)."""
    if dtype == "bf16":
        return bf16_to_f32(x).astype(np.float64)
    return np.asarray(x).astype(np.float64)


def combine(dtype: str, op: str, acc: np.ndarray, x: np.ndarray) -> np.ndarray:
    """rnd(acc (op) x), elementwise, in the buffer type.  ``acc`` is the
    left operand (the value already held), ``x`` the one folded in."""
    acc = np.asarray(acc)
    x = np.asarray(x)
    if op == "sum":
        if dtype == "i32":
            return (acc.astype(np.int64) + x.astype(np.int64)).astype(np.int32)
        if dtype == "i64":
            return (acc.view(np.uint64) + x.view(np.uint64)).view(np.int64)
        if dtype == "f32":
            return np.add(acc, x, dtype=np.float32)
        if dtype == "f16":
            wide = np.add(acc.astype(np.float32), x.astype(np.float32), dtype=np.float32)
            return wide.astype(np.float16)
        if dtype == "bf16":
            wide = np.add(bf16_to_f32(acc), bf16_to_f32(x), dtype=np.float32)
            return f32_to_bf16(wide)
    elif op == "max":
        if dtype in ("i32", "i64"):
            return np.maximum(acc, x)
        a = to_f64(acc, dtype)
        b = to_f64(x, dtype)
        take_x = (b > a) | ((b == a) & np.signbit(a) & ~np.signbit(b))
        return np.where(take_x, x, acc)
    raise ValueError(f"unknown dtype/op {dtype}/{op}")
