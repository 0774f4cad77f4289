"""Pins of the oracle on IEEE special values (subnormals, signed zeros,
overflow to infinity, infinities), for the ring and the tree on several
shapes.  Each pin follows from IEEE arithmetic and the construction of the
inputs, not from the oracle's code:

* a position whose inputs are all subnormals or zeros with small
  significands: every partial sum is a multiple of the smallest subnormal
  below the normal range, so every add is exact and the result is the exact
  integer sum of the signed significands (in units of the smallest
  subnormal); a zero result is -0 exactly when every input is -0;
* a position where two inputs lie in the largest finite binade with one
  sign, and no input has the other sign's infinity or large magnitude: the
  true sum exceeds the largest finite value, so once both are folded in the
  partial sum is an infinity of that sign and stays one;
* a position holding an infinity of one sign and no infinity of the other:
  the sum is that infinity;
* max: the largest value in the order of the reals with -0 below +0,
  computed here with Python floats.
"""

import math

import numpy as np
import pytest

from double_binary_tree_amd import inputs as I
from oracle import allreduce as A

LAYOUT = {"f32": (32, 8, 23), "f16": (16, 5, 10), "bf16": (16, 8, 7)}

SHAPES = [(1, 1, 1), (2, 1, 2), (6, 3, 3), (8, 1, 4), (16, 16, 2), (15, 15, 3), (32, 4, 2)]


def _bits(x, dtype):
    return np.ascontiguousarray(x).view(np.uint32 if dtype == "f32" else np.uint16).astype(np.int64)


def _fields(bits, dtype):
    width, ebits, mbits = LAYOUT[dtype]
    sign = (bits >> (width - 1)) & 1
    exp = (bits >> mbits) & ((1 << ebits) - 1)
    mant = bits & ((1 << mbits) - 1)
    return sign, exp, mant


def _value(bits, dtype):
    """Exact value of one element as a Python float (f32/f16/bf16 all fit a double)."""
    width, ebits, mbits = LAYOUT[dtype]
    s, e, m = (int(v) for v in _fields(np.int64(bits), dtype))
    bias = (1 << (ebits - 1)) - 1
    if e == (1 << ebits) - 1:
        assert m == 0, "no NaN expected"
        return -math.inf if s else math.inf
    mag = math.ldexp(m, 1 - bias - mbits) if e == 0 else math.ldexp((1 << mbits) | m, e - bias - mbits)
    return -mag if s else mag


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_special_inputs_are_as_documented(dtype):
    n = 8
    xs, cls, sign = I.special_inputs(n, dtype, 4000, seed=3)
    width, ebits, mbits = LAYOUT[dtype]
    emax = (1 << ebits) - 1
    b = np.stack([_bits(x, dtype) for x in xs])
    s, e, m = _fields(b, dtype)
    assert not ((e == emax) & (m != 0)).any(), "NaN in the inputs"
    tiny = cls == I.SPECIAL_TINY
    assert (e[:, tiny] == 0).all() and (m[:, tiny] < (1 << max(mbits - 6, 1))).all()
    for c in range(4):
        assert (cls == c).sum() > 800
    huge = (e == emax - 1)
    inf = (e == emax) & (m == 0)
    big = huge | inf
    # large magnitudes and infinities only with the position's sign
    assert not (big & (s != sign[None, :])).any()
    assert (huge.sum(axis=0)[cls == I.SPECIAL_HUGE] >= 2).all()
    assert (inf.sum(axis=0)[cls == I.SPECIAL_INF] >= 1).all()
    assert not big[:, (cls == I.SPECIAL_TINY) | (cls == I.SPECIAL_MIXED)].any()


@pytest.mark.parametrize("n,m,nch", SHAPES)
@pytest.mark.parametrize("algo", ["ring", "tree"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_oracle_sum_on_special_values(n, m, nch, algo, dtype):
    count = 1500 + 7
    xs, cls, sign = I.special_inputs(n, dtype, count, seed=n * 10 + nch)
    out = A.allreduce(xs, m, algo, nch, 64, dtype, "sum")
    width, ebits, mbits = LAYOUT[dtype]
    emax = (1 << ebits) - 1
    rb = _bits(out[0], dtype)
    for r in range(1, n):
        assert np.array_equal(_bits(out[r], dtype), rb)
    ib = np.stack([_bits(x, dtype) for x in xs])
    s, e, mant = _fields(ib, dtype)
    # tiny: exact sum of signed significands, -0 only from all -0
    tiny = np.nonzero(cls == I.SPECIAL_TINY)[0]
    total = (np.where(s == 1, -mant, mant)).sum(axis=0)
    for p in tiny:
        t = int(total[p])
        if t == 0:
            all_neg_zero = bool(((s[:, p] == 1) & (mant[:, p] == 0)).all())
            want = (1 << (width - 1)) if all_neg_zero else 0
        else:
            assert abs(t) < (1 << mbits), "construction keeps tiny sums subnormal"
            want = ((1 << (width - 1)) if t < 0 else 0) | abs(t)
        assert int(rb[p]) == want, (p, hex(int(rb[p])), hex(want))
    # huge and infinite positions: an infinity of the position's sign
    inf_bits = np.where(sign == 1, (1 << (width - 1)) | (emax << mbits), emax << mbits)
    for c in (I.SPECIAL_HUGE, I.SPECIAL_INF):
        sel = cls == c
        assert np.array_equal(rb[sel], inf_bits[sel]), c
    # mixed: finite, and within the forward error bound of the exact sum
    mixed = np.nonzero(cls == I.SPECIAL_MIXED)[0]
    u = math.ldexp(1.0, -(mbits + 1))
    for p in mixed[:300]:
        vals = [_value(int(ib[r, p]), dtype) for r in range(n)]
        got = _value(int(rb[p]), dtype)
        assert math.isfinite(got)
        exact = math.fsum(vals)
        bound = (n - 1) * u * math.fsum(abs(v) for v in vals) * (1 + n * u) + math.ldexp(n, 1 - ((1 << (ebits - 1)) - 1) - mbits)
        assert abs(got - exact) <= bound, (p, got, exact, bound)


@pytest.mark.parametrize("n,m,nch", SHAPES)
@pytest.mark.parametrize("algo", ["ring", "tree"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_oracle_max_on_special_values(n, m, nch, algo, dtype):
    count = 900 + 5
    xs, cls, sign = I.special_inputs(n, dtype, count, seed=500 + n * 10 + nch)
    out = A.allreduce(xs, m, algo, nch, 64, dtype, "max")
    ib = np.stack([_bits(x, dtype) for x in xs])
    rb = _bits(out[0], dtype)
    width = LAYOUT[dtype][0]
    for p in range(count):
        # the largest real value; among zeros, +0 above -0
        best = max(range(n), key=lambda r: (_value(int(ib[r, p]), dtype), not (int(ib[r, p]) >> (width - 1)) & 1))
        assert int(rb[p]) == int(ib[best, p]), (p, hex(int(rb[p])), hex(int(ib[best, p])))
