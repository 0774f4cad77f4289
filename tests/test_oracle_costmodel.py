"""Pins of the cost-model and selection oracle (CPU only)."""

import math

import pytest

from oracle import costmodel as C
from tests.conftest import golden_lines

UNITS = {"B": 1, "KiB": 1 << 10, "MiB": 1 << 20, "GiB": 1 << 30}
LADDER = [1 << p for p in range(2, 31)]          # 4 B .. 1 GiB


def _size(txt):
    for u in ("KiB", "MiB", "GiB", "B"):
        if txt.endswith(u):
            return int(txt[:-len(u)]) * UNITS[u]
    raise ValueError(txt)


def _rows(kind):
    return [ln.split()[1:] for ln in golden_lines("crossover_table.txt") if ln.split()[0] == kind]


def test_selected_points_relative_verdict_busbw():
    # "选定性能点": Tree relative to Ring, the tie verdict, and busbw of both.
    table = {}
    for n, w, a, b, pts, med, mx in _rows("INTERVAL"):
        table.setdefault(int(n), []).append((w, _size(a), _size(b)))
    for n, size, ring_us, tree_us, rel, rbus, tbus in _rows("POINT"):
        n, s, tr, tt = int(n), _size(size), float(ring_us), float(tree_us)
        assert round(100 * C.relative(tt, tr), 2) == pytest.approx(float(rel), abs=0.006)
        want = next(w for w, lo, hi in table[n] if lo <= s <= hi)
        assert C.verdict(tr, tt) == want, (n, size)
        # busbw of the median time; the page prints a median of per-sample
        # busbw over 10 samples (the mean of the middle two), which can differ
        # in the last printed digit
        assert round(C.busbw(s, tr * 1e-6, n) / 1e9, 2) == pytest.approx(float(rbus), abs=0.011)
        assert round(C.busbw(s, tt * 1e-6, n) / 1e9, 2) == pytest.approx(float(tbus), abs=0.011)


def test_crossover_table_is_a_merge_of_tie_rule_verdicts():
    # Every N's intervals cover the 4 B .. 1 GiB ladder in order; the point
    # counts are the ladder sizes inside each interval; a tie's largest
    # margin is under 5% and a winner's median margin is not; merging the
    # per-size verdicts gives back the intervals.
    by_n = {}
    for n, w, a, b, pts, med, mx in _rows("INTERVAL"):
        by_n.setdefault(int(n), []).append((w, _size(a), _size(b), int(pts), float(med), float(mx)))
    assert sorted(by_n) == [2, 3, 4]
    for n, rows in by_n.items():
        verdicts = []
        for w, lo, hi, pts, med, mx in rows:
            inside = [s for s in LADDER if lo <= s <= hi]
            assert len(inside) == pts, (n, w, lo, hi)
            if w == "Tie":
                assert mx / 100 < C.TIE
            else:
                assert med / 100 >= C.TIE
            verdicts += [w] * pts
        assert len(verdicts) == len(LADDER)
        merged = C.intervals(LADDER, verdicts)
        assert [(w, lo, hi, pts) for w, lo, hi, pts, _, _ in rows] == merged


def test_margin_of_the_tree_point_is_the_intervals_max():
    # N=2, 256 KiB: tree 6.85% faster means ring/tree - 1 = 7.35%, the
    # printed max margin of the N=2 tree interval.
    p = next(r for r in _rows("POINT") if r[0] == "2" and r[1] == "256KiB")
    m = C.margin(float(p[2]), float(p[3]))
    assert round(100 * m, 2) == 7.35


def test_closed_forms():
    # Interview page: each rank sends 2(n-1)/n * S, 1.5 S at n = 4; ring
    # 2(n-1) steps, 2046 at n = 1024; tree 2 log2 n, about 20.
    assert C.ring_time(4, 1000.0, alpha=0.0, bw=1.0) == 1500.0
    assert C.ring_stages(1024) == 2046
    assert C.tree_stages(int(math.log2(1024))) == 20
    assert C.tree_time(3, 1000.0, alpha=2.0, bw=4.0) == 6 * 2.0 + 500.0
    assert C.ring_time(8, 0.0, alpha=1.5, bw=1.0, launch=3.0) == 3.0 + 14 * 1.5


@pytest.mark.parametrize("n,depth", [(8, 7), (16, 4), (32, 9), (4, 3)])
def test_fit_recovers_the_model_parameters(n, depth):
    launch = 4.0
    ring = (0.35, 900.0, launch)     # alpha (us), bandwidth (bytes/us), launch (us)
    tree = (0.5, 1300.0, launch)
    sizes = [1 << p for p in range(3, 28)]
    for algo, (al, bw, la) in (("ring", ring), ("tree", tree)):
        f = (lambda s: C.ring_time(n, s, al, bw, la)) if algo == "ring" else (lambda s: C.tree_time(depth, s, al, bw, la))
        a, b = C.fit_line(sizes, [f(s) for s in sizes])
        alpha, bw_fit = C.params_from_fit(algo, n, depth, a, b, launch)
        assert alpha == pytest.approx(al, rel=1e-9)
        assert bw_fit == pytest.approx(bw, rel=1e-9)


def test_crossover_and_selection_agree():
    n, depth = 8, 3
    ring, tree = (0.4, 800.0, 5.0), (0.3, 500.0, 5.0)   # tree: fewer stages, lower bandwidth
    x = C.crossover(n, depth, ring, tree)
    assert x is not None and x > 0
    assert C.ring_time(n, x, *ring) == pytest.approx(C.tree_time(depth, x, *tree), rel=1e-12)
    assert C.select(n, depth, x * 0.5, ring, tree) == "tree"
    assert C.select(n, depth, x * 2.0, ring, tree) == "ring"
    # equal times choose the ring
    assert C.select(2, 1, 0.0, (1.0, 1.0, 0.0), (1.0, 1.0, 0.0)) == "ring"
