"""Pins of the oracle arithmetic (CPU only).

* bf16 rounding against the nearest point of the complete sorted grid of
  bf16 values (a search, not the bit rule the oracle uses);
* the 16-bit sums against the exactly rounded rational sum (Python
  fractions), which is what a correctly rounded 16-bit add means;
* float32 sum against Python's float64 sum rounded once (exact here);
* max against numpy.maximum and the +0/-0 convention;
* integer wrap-around against Python integers."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import numerics as N

ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _bf16_grid():
    vals = N.bf16_to_f32(ALL_BF16).astype(np.float64)
    finite = np.isfinite(vals)
    bits = ALL_BF16[finite]
    vals = vals[finite]
    order = np.argsort(vals, kind="stable")
    vals, bits = vals[order], bits[order]
    # Drop -0 (keep +0) so the grid is strictly increasing.
    keep = np.ones(len(vals), dtype=bool)
    keep[1:] = vals[1:] != vals[:-1]
    return vals[keep], bits[keep]


def _nearest_on_grid(x64, grid_vals, grid_bits):
    """Round-to-nearest-even by searching the sorted grid (values that lie
    past the largest finite bf16 by half an ulp or more become infinity)."""
    out = np.empty(len(x64), dtype=np.uint16)
    big = float(grid_vals[-1])
    ulp_top = big - float(grid_vals[-2])
    for i, x in enumerate(x64):
        if x >= big + ulp_top / 2:
            out[i] = 0x7F80
            continue
        if x <= -(big + ulp_top / 2):
            out[i] = 0xFF80
            continue
        j = int(np.searchsorted(grid_vals, x))
        lo = max(j - 1, 0)
        hi = min(j, len(grid_vals) - 1)
        if grid_vals[hi] == x and x != 0.0:
            out[i] = grid_bits[hi]
            continue
        dlo, dhi = x - grid_vals[lo], grid_vals[hi] - x
        if dlo < dhi:
            k = lo
        elif dhi < dlo:
            k = hi
        else:
            k = lo if grid_bits[lo] % 2 == 0 else hi
        out[i] = grid_bits[k]
        if grid_vals[k] == 0.0:
            # A value that rounds to zero keeps its sign.
            out[i] = 0x8000 if np.signbit(x) else 0x0000
    return out


def test_bf16_rounding_against_grid_search():
    rng = np.random.default_rng(1)
    grid_vals, grid_bits = _bf16_grid()
    # Random bit patterns over the whole finite float32 range, plus values
    # exactly halfway between neighbouring bf16 values, plus subnormals.
    u = rng.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    halfway = (rng.integers(0, 1 << 16, size=4000, dtype=np.uint64).astype(np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    sub = rng.integers(0, 1 << 23, size=2000, dtype=np.uint64).astype(np.uint32)
    u = np.concatenate([u, halfway, sub, sub | np.uint32(0x80000000),
                        np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00008000, 0x00018000], dtype=np.uint32)])
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    got = N.f32_to_bf16(x)
    want = _nearest_on_grid(x.astype(np.float64), grid_vals, grid_bits)
    assert np.array_equal(got, want)


def test_bf16_round_trip_and_specials():
    # Every bf16 value is a float32 value, so widening then rounding is exact.
    widened = N.bf16_to_f32(ALL_BF16)
    back = N.f32_to_bf16(widened)
    nan = np.isnan(widened)
    assert np.array_equal(back[~nan], ALL_BF16[~nan])
    assert np.all(np.isnan(N.bf16_to_f32(back[nan])))
    assert N.f32_to_bf16(np.array([np.inf, -np.inf], np.float32)).tolist() == [0x7F80, 0xFF80]


def _all_f16_sorted():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    ok = np.isfinite(vals)
    vals, bits = vals[ok], bits[ok]
    order = np.argsort(vals, kind="stable")
    vals, bits = vals[order], bits[order]
    keep = np.ones(len(vals), dtype=bool)
    keep[1:] = vals[1:] != vals[:-1]
    return vals[keep], bits[keep]


def _round_fraction_on_grid(fr, grid_vals, grid_bits, inf_bits):
    """Nearest-even rounding of an exact rational onto a sorted grid."""
    big = Fraction(float(grid_vals[-1]))
    half_ulp = (big - Fraction(float(grid_vals[-2]))) / 2
    if fr >= big + half_ulp:
        return inf_bits[0]
    if fr <= -(big + half_ulp):
        return inf_bits[1]
    j = int(np.searchsorted(grid_vals, float(fr)))
    best = None
    for k in (j - 2, j - 1, j, j + 1):
        if 0 <= k < len(grid_vals):
            d = abs(Fraction(float(grid_vals[k])) - fr)
            if best is None or d < best[0] or (d == best[0] and grid_bits[k] % 2 == 0):
                best = (d, grid_bits[k])
    return best[1]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_16bit_sum_is_correctly_rounded(dtype):
    rng = np.random.default_rng(2)
    if dtype == "f16":
        grid_vals, grid_bits = _all_f16_sorted()
        inf_bits = (0x7C00, 0xFC00)
        a_bits = rng.integers(0, 1 << 16, size=3000, dtype=np.uint64).astype(np.uint16)
        b_bits = rng.integers(0, 1 << 16, size=3000, dtype=np.uint64).astype(np.uint16)
        # Bias half the pairs towards close magnitudes (cancellation, ties).
        b_bits[:1500] = (a_bits[:1500] ^ rng.integers(0, 64, size=1500).astype(np.uint16)) ^ np.uint16(0x8000)
        a = a_bits.view(np.float16)
        b = b_bits.view(np.float16)
        ok = np.isfinite(a) & np.isfinite(b)
        a, b = a[ok], b[ok]
        got = N.combine("f16", "sum", a, b).view(np.uint16)
        exact = [Fraction(float(x)) + Fraction(float(y)) for x, y in zip(a, b)]
    else:
        grid_vals, grid_bits = _bf16_grid()
        inf_bits = (0x7F80, 0xFF80)
        a = rng.integers(0, 1 << 16, size=3000, dtype=np.uint64).astype(np.uint16)
        b = rng.integers(0, 1 << 16, size=3000, dtype=np.uint64).astype(np.uint16)
        b[:1500] = (a[:1500] ^ rng.integers(0, 64, size=1500).astype(np.uint16)) ^ np.uint16(0x8000)
        fa, fb = N.bf16_to_f32(a), N.bf16_to_f32(b)
        ok = np.isfinite(fa) & np.isfinite(fb)
        a, b, fa, fb = a[ok], b[ok], fa[ok], fb[ok]
        got = N.combine("bf16", "sum", a, b)
        exact = [Fraction(float(x)) + Fraction(float(y)) for x, y in zip(fa, fb)]
    for g, fr in zip(got, exact):
        want = _round_fraction_on_grid(fr, grid_vals, grid_bits, inf_bits)
        if fr == 0:
            assert g in (0x0000, 0x8000)
        else:
            assert int(g) == int(want), (fr, hex(int(g)), hex(int(want)))


def test_f32_sum_single_rounding():
    # Two float32 values: their exact sum fits in float64, so rounding the
    # float64 sum once to float32 is the correctly rounded float32 add.
    rng = np.random.default_rng(4)
    a = rng.standard_normal(10000).astype(np.float32) * np.float32(1e3)
    b = rng.standard_normal(10000).astype(np.float32)
    got = N.combine("f32", "sum", a, b)
    want = (a.astype(np.float64) + b.astype(np.float64)).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_integer_sums_wrap():
    big32 = np.array([2**31 - 1, -2**31], dtype=np.int32)
    one = np.array([1, -1], dtype=np.int32)
    assert N.combine("i32", "sum", big32, one).tolist() == [-2**31, 2**31 - 1]
    big64 = np.array([2**63 - 1], dtype=np.int64)
    assert N.combine("i64", "sum", big64, np.array([1], np.int64)).tolist() == [-2**63]
    rng = np.random.default_rng(5)
    a = rng.integers(-2**40, 2**40, size=1000)
    b = rng.integers(-2**40, 2**40, size=1000)
    assert N.combine("i64", "sum", a, b).tolist() == [int(x) + int(y) for x, y in zip(a, b)]


@pytest.mark.parametrize("dtype", ["i32", "i64", "f32", "f16"])
def test_max_matches_numpy(dtype):
    rng = np.random.default_rng(6)
    if dtype.startswith("i"):
        a = rng.integers(-1000, 1000, size=5000).astype(N.STORAGE[dtype])
        b = rng.integers(-1000, 1000, size=5000).astype(N.STORAGE[dtype])
    else:
        a = rng.standard_normal(5000).astype(N.STORAGE[dtype])
        b = rng.standard_normal(5000).astype(N.STORAGE[dtype])
    assert np.array_equal(N.combine(dtype, "max", a, b), np.maximum(a, b))


def test_max_bf16_and_signed_zero():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(4000).astype(np.float32)
    y = rng.standard_normal(4000).astype(np.float32)
    a, b = N.f32_to_bf16(x), N.f32_to_bf16(y)
    got = N.bf16_to_f32(N.combine("bf16", "max", a, b))
    assert np.array_equal(got, np.maximum(N.bf16_to_f32(a), N.bf16_to_f32(b)))
    pz, nz = np.array([0.0], np.float32), np.array([-0.0], np.float32)
    for acc, x in ((pz, nz), (nz, pz)):
        assert not np.signbit(N.combine("f32", "max", acc, x))[0]
