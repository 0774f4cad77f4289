"""Pins of the oracle partition (CPU only).

The split rule itself is a reading (the pages name the fields only), so the
pins are invariants that any mistake in it would break, plus the one case
the pages do fix: with a unit of one element the ring's rank-chunks are
``numpy.array_split``'s parts (interview page, section "手撕代码")."""

import itertools

import numpy as np
import pytest

from oracle import partition as P


def _covers(ranges, start, end):
    pos = start
    for o, ln in ranges:
        assert o == pos and ln >= 0
        pos += ln
    assert pos == end


@pytest.mark.parametrize("unit", [1, 2, 4, 8])
def test_channel_ranges_cover_disjoint_aligned(unit):
    for count in list(range(0, 70)) + [1000, 1023, 4097, 65537]:
        for nch in (1, 2, 3, 5, 12, 32, 64):
            ranges = P.channel_ranges(count, unit, nch)
            assert len(ranges) == nch
            _covers(ranges, 0, count)
            sizes_units = [-(-ln // unit) for _, ln in ranges]
            assert max(sizes_units) - min(sizes_units) <= 1
            for o, ln in ranges:
                assert o % unit == 0 or o == count
                if o + ln != count:
                    assert ln % unit == 0
            # Larger parts first (array_split order).
            assert all(a >= b for a, b in zip(sizes_units, sizes_units[1:]) if b)


def test_tree_chunks():
    for off, cnt, ck in itertools.product((0, 16, 100), (0, 1, 7, 64, 65, 1000), (1, 4, 64)):
        chunks = P.tree_chunks(off, cnt, ck)
        _covers(chunks, off, off + cnt)
        assert all(ln == ck for _, ln in chunks[:-1])
        assert len(chunks) == -(-cnt // ck)


def test_ring_loops_unit_one_is_array_split():
    rng = np.random.default_rng(7)
    for n in range(1, 10):
        for length in list(range(0, 40)) + [97, 128]:
            x = rng.standard_normal(length)
            loops = P.ring_loops(0, length, n, chunk_count=max(1, length), unit=1)
            if length == 0:
                assert loops == []
                continue
            assert len(loops) == 1
            parts = np.array_split(x, n)
            assert [ln for _, ln in loops[0]] == [len(p) for p in parts]


@pytest.mark.parametrize("unit", [1, 2, 4])
def test_ring_loops_cover_and_split(unit):
    for n in (1, 2, 3, 4, 8):
        for ck in (unit, 2 * unit, 8 * unit):
            for cnt in (0, 1, unit - 1, unit, unit + 1, n * ck - 1, n * ck, n * ck + 1, 3 * n * ck + 5):
                if cnt < 0:
                    continue
                loops = P.ring_loops(64, cnt, n, ck, unit)
                flat = [b for lp in loops for b in lp]
                _covers(flat, 64, 64 + cnt)
                for lp in loops:
                    assert len(lp) == n
                    assert sum(ln for _, ln in lp) <= n * ck
                for lp in loops[:-1]:
                    assert all(ln == ck for _, ln in lp)


def test_channel_example_twelve_channels():
    # 16 Mi float32 elements over 12 channels in 16-byte units: 4,194,304
    # units, 349,525 each plus one more for the first four channels.
    ranges = P.channel_ranges(16 * 1024 * 1024, 4, 12)
    assert [ln for _, ln in ranges] == [1398104] * 4 + [1398100] * 8
