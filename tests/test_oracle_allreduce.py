"""Pins of the whole oracle all-reduce (CPU only): brute force on tiny
inputs, the float64 bound, in-place equivalence and the sampled variant."""

import itertools

import numpy as np
import pytest

from double_binary_tree_amd import inputs as I
from oracle import allreduce as A
from oracle import numerics as N


def _draw(n, count, dtype, seed):
    rng = np.random.default_rng(seed)
    if dtype == "i32":
        return [rng.integers(-1000, 1001, size=count).astype(np.int32) for _ in range(n)]
    if dtype == "i64":
        return [rng.integers(-(1 << 40), (1 << 40) + 1, size=count).astype(np.int64) for _ in range(n)]
    x = [rng.standard_normal(count).astype(np.float32) for _ in range(n)]
    if dtype == "f32":
        return x
    if dtype == "f16":
        return [(v * np.float32(0.1)).astype(np.float16) for v in x]
    return [N.f32_to_bf16(v) for v in x]


def _counts(n, unit):
    return sorted({0, 1, unit - 1, unit, unit + 1, n * unit - 1, n * unit, n * unit + 1,
                   3 * n * unit + 3} - {-1})


def _shapes():
    for n in range(1, 10):
        for m in range(1, n + 1):
            if n % m == 0:
                yield n, m


def test_brute_force_integer_and_max():
    # Integer sums and every max must be the plain reduction, whatever the
    # schedule; every rank must hold the same bits.
    cases = 0
    for (n, m), nch, algo in itertools.product(_shapes(), (1, 2, 4), ("ring", "tree")):
        for dtype, op in (("i32", "sum"), ("i64", "max"), ("f32", "max")):
            unit = 16 // N.ITEMSIZE[dtype]
            for count in _counts(n, unit):
                xs = _draw(n, count, dtype, seed=cases)
                chunk = 2 * 16  # two units per chunk: many chunks and loops
                out = A.allreduce(xs, m, algo, nch, chunk, dtype, op)
                if op == "sum":
                    want = A.reference_sum(xs, dtype)
                    assert [int(v) for v in out[0]] == [int(v) for v in want]
                else:
                    want = np.max(np.stack(xs), axis=0) if count else np.zeros(0, xs[0].dtype)
                    assert np.array_equal(out[0], want)
                for o in out[1:]:
                    assert np.array_equal(o.view(np.uint8), out[0].view(np.uint8))
                cases += 1
    assert cases > 1000


@pytest.mark.parametrize("dtype,rtol", [("f32", 1e-5), ("f16", 1e-2), ("bf16", 1e-2)])
def test_float_sums_within_fp64_bound(dtype, rtol):
    for (n, m), nch, algo in itertools.product([(2, 1), (3, 3), (4, 2), (8, 1), (9, 3)], (1, 3),
                                               ("ring", "tree")):
        xs = _draw(n, 1000, dtype, seed=n * 7 + nch)
        out = A.allreduce(xs, m, algo, nch, 64, dtype, "sum")
        ok, worst = A.within_tolerance(out[0], xs, dtype, rtol)
        assert ok, (n, m, nch, algo, worst)
        ok, worst = A.within_rounding_bound(out[0], xs, dtype)
        assert ok, (n, m, nch, algo, worst)
        for o in out[1:]:
            assert np.array_equal(o.view(np.uint8), out[0].view(np.uint8))


def test_rounding_bound_catches_a_dropped_term():
    # The elementwise bound is tight enough that losing one rank's input
    # (a plausible oracle mistake) fails it.
    xs = _draw(4, 500, "bf16", seed=3)
    out = A.allreduce(xs, 1, "ring", 1, 64, "bf16", "sum")
    assert A.within_rounding_bound(out[0], xs, "bf16")[0]
    assert not A.within_rounding_bound(out[0], xs[:3] + [N.f32_to_bf16(np.zeros(500, np.float32))],
                                       "bf16")[0]


def test_inputs_left_untouched_and_inplace_equivalent():
    # The oracle never writes its inputs, so an in-place call (outputs
    # overwriting inputs) has the same values as an out-of-place one.
    xs = _draw(5, 333, "f32", seed=11)
    keep = [x.copy() for x in xs]
    A.allreduce(xs, 5, "tree", 3, 64, "f32", "sum")
    A.allreduce(xs, 1, "ring", 3, 64, "f32", "sum")
    for a, b in zip(xs, keep):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ["chain8_f32", "dtree16_bf16", "dtree15_bf16", "hier4x8_f16",
                                  "hier4x8_i64", "hier4x8_f32max", "ring4_i32"])
def test_sampled_equals_full(name):
    w = I.WORKLOADS[name]
    count = 3 * 4096 + 5
    xs = I.rank_inputs(w, count=count)
    chunk = 1024  # small chunks so that the reduced size still has many loops
    rng = np.random.default_rng(0)
    idx = np.unique(np.concatenate([rng.integers(0, count, size=300), [0, count - 1]]))
    for algo in w.algos:
        full = A.allreduce(xs, w.nnodes, algo, w.nchannels, chunk, w.dtype, w.op)
        part = A.allreduce_at(xs, idx, w.nnodes, algo, w.nchannels, chunk, w.dtype, w.op)
        assert np.array_equal(full[0][idx].view(np.uint8), part.view(np.uint8))


def test_workload_inputs_are_seeded_and_shaped():
    w = I.WORKLOADS["hier4x8_f16"]
    a = I.rank_inputs(w, count=100)
    b = I.rank_inputs(w, count=100)
    assert len(a) == 32 and all(x.dtype == np.float16 and len(x) == 100 for x in a)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert not np.array_equal(a[0], a[1])
